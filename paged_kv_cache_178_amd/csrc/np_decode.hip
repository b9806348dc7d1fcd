// Split-KV paged-attention decode for gfx950 (MI355X), plus the split combine.
//
// What is computed ("I Wrote the Three Attention Kernels That Run LLM
// Inference -- in Portable Triton, on a Free Colab T4"; sections "What is
// attention, really?", "2. Split-KV flash-decoding", "3. Paged KV-cache
// attention"): for each sequence s and query head h,
//   out[s,h,:] = sum_t softmax_t(scale <q[s,h,:], K[t]>) V[t],
// with K[t], V[t] read from slot t % B of physical block table[s, t / B], KV
// head h / G (G = Hq/Hkv). The KV range of a sequence may be cut into splits;
// each split yields (m, l, acc) and the combine kernel merges them with the
// log-sum-exp weights of the split-KV page.
//
// Work decomposition (MI355X-first, not the pages' one-program-per-head grid):
// * One 256-thread workgroup (4 wave64) per (sequence, KV head, split). All G
//   query heads of the GQA group are computed from each K/V row while it is in
//   registers, so the KV stream is read from HBM exactly once.
// * A K or V row of one head (d_pad channels) is covered by LPR lanes with one
//   16-byte load each (8 lanes x 16 B = 128 B for bf16/fp16 d=64, one cache
//   line). One wave load therefore covers TPL = 64/LPR consecutive slots.
// * Waves take whole blocks round-robin and issue all K/V loads of a group of
//   blocks before computing any of them.
// * The lanes of a row each hold VEC channels of one slot; the only
//   cross-lane work per block is the LPR-lane sum of the QK partial dot
//   products (DPP). Weights and V of two slots are packed so P.V is a v_dot2.
// * Scores of a group of blocks are computed first; the wave-wide max of the
//   group moves the running max once, so earlier sums are rescaled once per
//   group and the block bodies carry no branches.
// * The online-softmax max is shared by a whole wave, so at the end the rows
//   of a wave add directly and the waves are merged through LDS.
// Scores are kept in log2 units (scale * log2 e folded in), exp2 is v_exp_f32.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "np_internal.h"
#include "np_table.h"

namespace np {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* bt;
  const int32_t* lens;
  void* out;
  uint32_t* ws_cnt;
  float* ws_ml;
  float* ws_acc;
  int64_t q_s0, q_s1;
  int64_t kv_s0, kv_s1, kv_s2;
  int64_t o_s0, o_s1;
  int64_t bt_stride;
  int32_t bt_contig;             // 1: NULL table, contiguous layout
  int32_t hkv, hq, head_dim, max_blocks, bps, max_splits;
  int32_t num_seqs;
  int32_t sk_cost;   // stream-K: virtual units per segment
  float scale_log2;
  int32_t* trace;    // trace build only (NP_TRACE): per-workgroup records
};

// ------------------------------------------------------------- trace build
//
// Compiled with NP_TRACE (the debugging and measurement library
// libnp_paged_trace.so, never the product library), the decode kernels write
// one record per workgroup into the buffer registered with
// np_debug_set_trace: the uniform-split kernel its coordinates and the
// s_memrealtime time of each phase, the stream-K kernel the pieces it read
// and the partial slots it merged (layouts in np_trace.h). A stamp first
// waits for every outstanding memory operation of the wave, so the trace
// build's timing is that of a kernel without overlap across the stamped
// points. Without NP_TRACE the hooks are empty.
#ifdef NP_TRACE
struct Stamps {
  uint64_t t[kTraceStamps];
  __device__ __forceinline__ Stamps() {
#pragma unroll
    for (int i = 0; i < kTraceStamps; ++i) t[i] = 0;
  }
  __device__ __forceinline__ void at(int i) {
    __builtin_amdgcn_s_waitcnt(0);
    t[i] = __builtin_amdgcn_s_memrealtime();
  }
};
__device__ __forceinline__ int32_t trace_where() { return int32_t(__smid()); }
#else
struct Stamps {
  __device__ __forceinline__ void at(int) {}
};
#endif

// ------------------------------------------------------------ element types

template <int DT>
struct Elt;
template <>
struct Elt<NP_F32> {
  static constexpr int kBytes = 4;
};
template <>
struct Elt<NP_F16> {
  static constexpr int kBytes = 2;
};
template <>
struct Elt<NP_BF16> {
  static constexpr int kBytes = 2;
};

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

// Partial dot product of two 16-byte chunks (same element type), fp32 result.
template <int DT>
__device__ __forceinline__ float dot16(const uint4& a, const uint4& b, float c);

template <>
__device__ __forceinline__ float dot16<NP_BF16>(const uint4& a, const uint4& b, float c) {
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                      __builtin_bit_cast(bf16x2_t, b.x), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                      __builtin_bit_cast(bf16x2_t, b.y), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                      __builtin_bit_cast(bf16x2_t, b.z), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                      __builtin_bit_cast(bf16x2_t, b.w), c, false);
  return c;
}

template <>
__device__ __forceinline__ float dot16<NP_F16>(const uint4& a, const uint4& b, float c) {
  c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.x),
                             __builtin_bit_cast(f16x2_t, b.x), c, false);
  c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.y),
                             __builtin_bit_cast(f16x2_t, b.y), c, false);
  c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.z),
                             __builtin_bit_cast(f16x2_t, b.z), c, false);
  c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a.w),
                             __builtin_bit_cast(f16x2_t, b.w), c, false);
  return c;
}

template <>
__device__ __forceinline__ float dot16<NP_F32>(const uint4& a, const uint4& b, float c) {
  c = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), c);
  c = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), c);
  c = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), c);
  c = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), c);
  return c;
}

// Unpack a 16-byte chunk into fp32 values (the fp32 path; 16-bit types use
// packed v_dot2 on the raw words instead).
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& a, float* f);

template <>
__device__ __forceinline__ void unpack16<NP_F32>(const uint4& a, float* f) {
  f[0] = __uint_as_float(a.x);
  f[1] = __uint_as_float(a.y);
  f[2] = __uint_as_float(a.z);
  f[3] = __uint_as_float(a.w);
}

// Output rows hold head_dim channels, a multiple of 8 (16-bit types) or 4
// (fp32) by the 16-byte row rule the host checks, with rows and the base
// 16-byte aligned: a chunk of 2 or 4 channels starting at an even (multiple
// of 4) channel below head_dim is whole and aligned, so it is one store.
template <int DT>
__device__ __forceinline__ void store_out2(void* base, int64_t idx, float a, float b);
template <>
__device__ __forceinline__ void store_out2<NP_F32>(void* base, int64_t idx, float a, float b) {
  *reinterpret_cast<float2*>(static_cast<float*>(base) + idx) = make_float2(a, b);
}
template <>
__device__ __forceinline__ void store_out2<NP_F16>(void* base, int64_t idx, float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f2_t;
  const f2_t v = {a, b};
  *reinterpret_cast<f16x2_t*>(static_cast<_Float16*>(base) + idx) =
      __builtin_convertvector(v, f16x2_t);
}
template <>
__device__ __forceinline__ void store_out2<NP_BF16>(void* base, int64_t idx, float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f2_t;
  const f2_t v = {a, b};
  *reinterpret_cast<bf16x2_t*>(static_cast<__bf16*>(base) + idx) =
      __builtin_convertvector(v, bf16x2_t);
}
template <int DT>
__device__ __forceinline__ void store_out4(void* base, int64_t idx, float4 x) {
  if constexpr (DT == NP_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + idx) = x;
  } else {
    // Two packed pairs, one 8-byte store.
    typedef __attribute__((ext_vector_type(2))) float f2_t;
    const f2_t lo = {x.x, x.y}, hi = {x.z, x.w};
    uint2 w;
    if constexpr (DT == NP_BF16) {
      w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2_t));
      w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2_t));
      *reinterpret_cast<uint2*>(static_cast<__bf16*>(base) + idx) = w;
    } else {
      w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, f16x2_t));
      w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, f16x2_t));
      *reinterpret_cast<uint2*>(static_cast<_Float16*>(base) + idx) = w;
    }
  }
}

template <int DT>
__device__ __forceinline__ void store_out(void* base, int64_t idx, float x);
template <>
__device__ __forceinline__ void store_out<NP_F32>(void* base, int64_t idx, float x) {
  static_cast<float*>(base)[idx] = x;
}
template <>
__device__ __forceinline__ void store_out<NP_F16>(void* base, int64_t idx, float x) {
  static_cast<_Float16*>(base)[idx] = static_cast<_Float16>(x);
}
template <>
__device__ __forceinline__ void store_out<NP_BF16>(void* base, int64_t idx, float x) {
  static_cast<__bf16*>(base)[idx] = static_cast<__bf16>(x);
}

// Heads h0 .. h0 + n - 1 of sequence s's output row set to NaN (the whole
// workgroup takes part).
template <int DT, typename Params>
__device__ __forceinline__ void fill_nan(const Params& p, int s, int h0, int n) {
  for (int i = threadIdx.x; i < n * p.head_dim; i += blockDim.x)
    store_out<DT>(p.out, int64_t(s) * p.o_s0 + int64_t(h0 + i / p.head_dim) * p.o_s1 +
                             i % p.head_dim,
                  __builtin_nanf(""));
}

// ------------------------------------------------------- cross-lane helpers

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}

// Sum over the LPR consecutive lanes that share one K row. After the two quad
// steps every lane holds its quad's sum; half-row mirror pairs lane i with
// 7-i (the other quad of the 8-lane group), row mirror pairs i with 15-i.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (LPR >= 2) x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (LPR >= 4) x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) x += dpp_f<0x141>(x);  // row_half_mirror
  if constexpr (LPR >= 16) x += dpp_f<0x140>(x); // row_mirror
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

// Sum of N values (N a multiple of 4) over the 8 rows of a wave whose rows
// are 8 lanes wide (lane bits 3..5). Bit 3 is a DPP row rotate; bits 4 and 5
// use the gfx950 lane swaps, each of which exchanges half of two registers
// between lane groups, so one swap and one add reduce two values at once and
// leave them interleaved. On return u[k] holds, in 16-lane group r, value
// 4k + r summed over all 8 rows (lanes i and i ^ 8 hold the same sums).
template <int N>
__device__ __forceinline__ void rows8_sum(float (&v)[N], float (&u)[N / 4]) {
  static_assert(N % 4 == 0, "values come in fours");
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] += dpp_f<0x128>(v[k]);   // row_ror:8 (lane i <-> i^8)
  float w[N / 2];
#pragma unroll
  for (int j = 0; j < N / 2; ++j) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v[2 * j]),
                                                    __builtin_bit_cast(uint32_t, v[2 * j + 1]),
                                                    false, false);
    // (Elements copied out first: a bit cast applied to the subscripted
    // result reads element 0 twice with this compiler.)
    const uint32_t r0 = r[0], r1 = r[1];
    w[j] = __uint_as_float(r0) + __uint_as_float(r1);
  }
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, w[2 * k]),
                                                    __builtin_bit_cast(uint32_t, w[2 * k + 1]),
                                                    false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    u[k] = __uint_as_float(r0) + __uint_as_float(r1);
  }
}

__device__ __forceinline__ uint4 load16(const void* base, int64_t elem_off, int elt) {
  return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + elem_off * elt);
}

typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;

// K/V rows are read exactly once per call: a nontemporal (streaming) load
// keeps them from displacing reusable lines.
__device__ __forceinline__ uint4 load16_stream(const void* base, int64_t elem_off, int elt) {
  const u32x4_t v = __builtin_nontemporal_load(
      reinterpret_cast<const u32x4_t*>(static_cast<const char*>(base) + elem_off * elt));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Split partials are published with agent-scope relaxed atomic stores and
// read back with buffer loads that carry the device-scope cache bit (the bit
// an agent-scope atomic load carries). On gfx950 both are plain stores and
// loads with the device-coherence bit set, so the partials bypass the per-XCD
// L2 and no L2 write-back or invalidate (what an agent-scope fence costs, per
// workgroup) is needed. The writer waits for its stores to
// complete before it takes its arrival ticket; the reader issues its loads only
// after seeing that every other ticket was taken.
__device__ __forceinline__ void publish2(float* p, float a, float b) {
  const uint64_t v = uint64_t(__float_as_uint(a)) | (uint64_t(__float_as_uint(b)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Word 3 of a buffer descriptor for untyped loads: data format 32 bits
// (a zero format makes untyped buffer loads return 0), no swizzle, no index
// stride.
constexpr int kBufferWord3 = 0x00020000;
// Cache policy of a load that reads what other workgroups published with
// agent-scope stores: the device-scope bit (sc1), the same bit an agent-scope
// atomic load carries.
constexpr int kDeviceScopeLoad = 16;

// Merge the splits of one (sequence, KV head): with M = max_j m_j,
// out = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j. This is the split-KV
// page's log-sum-exp combine written with unnormalised partials
// (lse_j = m_j + log l_j, out_j = acc_j / l_j, in log2 units).
//
// Latency-parallel: waves take splits round-robin, each lane owns float4
// chunks of the G x d_pad output, and a batch of UB splits has all its loads
// in flight before any is used (one 16-byte acc load per split and chunk, one
// (m, l) load per wave); the per-wave states are merged through LDS.
// The partials of query head kvh * G + h and split j sit at part
// row0 + h * max_splits + j. Each lane's offset inside the head group's rows
// is computed once; a split moves every lane by the same amount, which is a
// scalar offset of a buffer load (one descriptor per head group), so issuing
// a split's loads costs no vector address arithmetic. Every read stays in
// the head group's rows: j < splits <= max_splits.
template <int DT, int D_PAD, int G>
__device__ __forceinline__ void merge_splits(const DecodeParams& p, int s, int kvh, int splits,
                                             bool write = true) {
  constexpr int NW = kDecodeWaves;
  constexpr int NCH = G * D_PAD / 4;          // float4 chunks of the output
  constexpr int CPL = (NCH + kWaveSize - 1) / kWaveSize;
  constexpr int UB = CPL > 1 ? 4 : 8;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int lane = threadIdx.x % kWaveSize;
  splits = __builtin_amdgcn_readfirstlane(splits);

  const int64_t row0 = (int64_t(s) * p.hq + int64_t(kvh) * G) * p.max_splits;
  const __amdgpu_buffer_rsrc_t r_acc = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<void*>(p.ws_acc + row0 * D_PAD), 0, G * p.max_splits * D_PAD * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t r_ml = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<void*>(p.ws_ml + 2 * row0), 0, G * p.max_splits * 8, kBufferWord3);
  int acc_off[CPL], hd[CPL];
#pragma unroll
  for (int ci = 0; ci < CPL; ++ci) {
    // Lanes past the output re-read its last chunk and get weight 0.
    const int chunk = lane + ci * kWaveSize;
    const int cc = chunk < NCH ? chunk : NCH - 1;
    hd[ci] = (cc * 4) / D_PAD;
    acc_off[ci] = (hd[ci] * p.max_splits * D_PAD + (cc * 4) % D_PAD) * 4;
  }
  // The (m, l) pairs of a batch: lane u * G + h of a wave loads split u's
  // pair of head h (UB * G <= 64 lanes), and every lane reads the pairs of
  // its chunks' heads back from the wave's LDS row. A full-width load costs
  // the CU's address unit about the same whatever it reads, and the time to
  // issue the batch is what the merge waits on, so one load here instead of
  // UB per lane shortens it.
  static_assert(UB * G <= kWaveSize, "a batch's (m, l) pairs fit one wave");
  __shared__ float2 s_mlb[NW][kWaveSize];
  const int pl = lane < UB * G ? lane : UB * G - 1;
  const int pu = pl / G, phd = pl % G;

  float mw[CPL], dw[CPL];
  float4 nw[CPL];
#pragma unroll
  for (int ci = 0; ci < CPL; ++ci) {
    mw[ci] = -INFINITY;
    dw[ci] = 0.0f;
    nw[ci] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int j0 = wave; j0 < splits; j0 += NW * UB) {
    float2 ml[UB][CPL];
    float4 a[UB][CPL];
    // A split past the last re-reads the last one and gets weight 0, so the
    // batch is issued without branches.
    const int jp = j0 + pu * NW < splits ? j0 + pu * NW : splits - 1;
    const u32x2_t mp = __builtin_amdgcn_raw_buffer_load_b64(
        r_ml, (phd * p.max_splits + jp) * 8, 0, kDeviceScopeLoad);
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int j = j0 + u * NW < splits ? j0 + u * NW : splits - 1;
#pragma unroll
      for (int ci = 0; ci < CPL; ++ci) {
        const u32x4_t a4 = __builtin_amdgcn_raw_buffer_load_b128(r_acc, acc_off[ci],
                                                                  j * D_PAD * 4, kDeviceScopeLoad);
        a[u][ci] = make_float4(__uint_as_float(a4.x), __uint_as_float(a4.y),
                               __uint_as_float(a4.z), __uint_as_float(a4.w));
      }
    }
    // Keep the whole batch of loads ahead of the first use: left to itself
    // the scheduler may sink the last split's loads below the maximum, which
    // costs one more memory round trip.
    __builtin_amdgcn_sched_barrier(0);
    // (The row is the wave's own: its lanes write and read it in program
    // order, which LDS keeps, so no barrier.)
    s_mlb[wave][lane] = make_float2(__uint_as_float(mp.x), __uint_as_float(mp.y));
#pragma unroll
    for (int u = 0; u < UB; ++u)
#pragma unroll
      for (int ci = 0; ci < CPL; ++ci) ml[u][ci] = s_mlb[wave][u * G + hd[ci]];
#pragma unroll
    for (int u = 0; u < UB; ++u)
#pragma unroll
      for (int ci = 0; ci < CPL; ++ci)
        if (j0 + u * NW >= splits || lane + ci * kWaveSize >= NCH) ml[u][ci].x = -INFINITY;
#pragma unroll
    for (int ci = 0; ci < CPL; ++ci) {
      float mx = mw[ci];
#pragma unroll
      for (int u = 0; u < UB; ++u) mx = fmaxf(mx, ml[u][ci].x);
      // A batch with no split in it (mx still -inf) must leave the state as
      // it is: its weights are then exp2(-inf) = 0. This is a select, not a
      // skip, so every load of the batch is consumed on every path. A load
      // left pending at the loop's back edge (as a skip leaves it) makes the
      // compiler guard its register at the top of the loop with a counter
      // wait placed among the batch's loads, which holds the last loads back
      // until the first ones have returned: a second memory round trip.
      const float ms = mx == -INFINITY ? 0.0f : mx;
      const float aw = __builtin_amdgcn_exp2f(mw[ci] - ms);
      float d = dw[ci] * aw;
      float4 n = make_float4(nw[ci].x * aw, nw[ci].y * aw, nw[ci].z * aw, nw[ci].w * aw);
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const float w = __builtin_amdgcn_exp2f(ml[u][ci].x - ms);
        d = fmaf(w, ml[u][ci].y, d);
        n.x = fmaf(w, a[u][ci].x, n.x);
        n.y = fmaf(w, a[u][ci].y, n.y);
        n.z = fmaf(w, a[u][ci].z, n.z);
        n.w = fmaf(w, a[u][ci].w, n.w);
      }
      mw[ci] = mx;
      dw[ci] = d;
      nw[ci] = n;
    }
  }
  __shared__ float s_m[NW][CPL * kWaveSize];
  __shared__ float s_d[NW][CPL * kWaveSize];
  __shared__ float4 s_n[NW][CPL * kWaveSize];
#pragma unroll
  for (int ci = 0; ci < CPL; ++ci) {
    s_m[wave][lane + ci * kWaveSize] = mw[ci];
    s_d[wave][lane + ci * kWaveSize] = dw[ci];
    s_n[wave][lane + ci * kWaveSize] = nw[ci];
  }
  __syncthreads();
  for (int chunk = threadIdx.x; chunk < NCH; chunk += blockDim.x) {
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_m[w][chunk]);
    float d = 0.0f;
    float4 n = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = __builtin_amdgcn_exp2f(s_m[w][chunk] - mx);   // 0 for idle waves
      d = fmaf(a, s_d[w][chunk], d);
      n.x = fmaf(a, s_n[w][chunk].x, n.x);
      n.y = fmaf(a, s_n[w][chunk].y, n.y);
      n.z = fmaf(a, s_n[w][chunk].z, n.z);
      n.w = fmaf(a, s_n[w][chunk].w, n.w);
    }
    const int h = (chunk * 4) / D_PAD;
    const int c = (chunk * 4) % D_PAD;
    const int64_t o = int64_t(s) * p.o_s0 + int64_t(kvh * G + h) * p.o_s1 + c;
    const float r = __builtin_amdgcn_rcpf(d);
    if (write && c < p.head_dim)
      store_out4<DT>(p.out, o, make_float4(n.x * r, n.y * r, n.z * r, n.w * r));
  }
}

// ------------------------------------------------------- math helpers

// Max over the rows of a wave (lanes that differ in the row index); the LPR
// lanes of one row already hold the same value. Result is wave-uniform.
template <int LPR>
__device__ __forceinline__ float wave_max_rows(float x) {
  if constexpr (LPR <= 8) x = fmaxf(x, dpp_f<0x128>(x));   // row_ror:8 (lane i <-> i^8)
  if constexpr (LPR <= 16) {
    // Lanes i and i ^ 16: a gfx950 lane swap of x with itself leaves, in
    // every lane, one 16-lane group of the pair in each result, so their max
    // is the pair's. (A VALU op: an LDS swizzle here would make the compiler
    // wait on the lgkm counter, which also waits for the scalar table reads
    // of the next group.)
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    x = fmaxf(__uint_as_float(r0), __uint_as_float(r1));
  }
  const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  return fmaxf(lo, hi);
}

// P.V for one pair of slots (ja, jb) held by this lane, 16-bit types: the two
// slots' V values of each channel are packed side by side (v_perm) and the
// two weights are rounded to the input type, so one v_dot2 adds both slots'
// contributions of a channel in fp32. The softmax denominator l adds the
// same rounded pair (a v_dot2 against (1, 1)), so numerator and denominator
// use identical weights.
template <int DT, int G, int VEC>
__device__ __forceinline__ void pv_pair(const uint4& va, const uint4& vb, const float (*w)[G],
                                        int ja, int jb, float (*acc)[VEC], float* l) {
  const uint32_t a[4] = {va.x, va.y, va.z, va.w};
  const uint32_t b[4] = {vb.x, vb.y, vb.z, vb.w};
  uint32_t pr[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    pr[2 * k] = __builtin_amdgcn_perm(b[k], a[k], 0x05040100u);       // low halves
    pr[2 * k + 1] = __builtin_amdgcn_perm(b[k], a[k], 0x07060302u);   // high halves
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    typedef __attribute__((ext_vector_type(2))) float f2_t;
    const f2_t ww = {w[ja][h], w[jb][h]};
    if constexpr (DT == NP_BF16) {
      const bf16x2_t wp = __builtin_convertvector(ww, bf16x2_t);
      l[h] = __builtin_amdgcn_fdot2_f32_bf16(wp, __builtin_bit_cast(bf16x2_t, 0x3f803f80u), l[h],
                                             false);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[h][c] = __builtin_amdgcn_fdot2_f32_bf16(wp, __builtin_bit_cast(bf16x2_t, pr[c]),
                                                    acc[h][c], false);
    } else {
      const f16x2_t wp = __builtin_convertvector(ww, f16x2_t);
      l[h] = __builtin_amdgcn_fdot2(wp, __builtin_bit_cast(f16x2_t, 0x3c003c00u), l[h], false);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[h][c] = __builtin_amdgcn_fdot2(wp, __builtin_bit_cast(f16x2_t, pr[c]), acc[h][c],
                                           false);
    }
  }
}

// ------------------------------------------------------------------ kernel

// Tile constants of one instantiation.
template <int DT, int D_PAD, int BS, int NWAVES = kDecodeWaves>
struct DecodeShape {
  static constexpr int kElt = Elt<DT>::kBytes;
  static constexpr int VEC = 16 / kElt;          // elements per lane-load
  static constexpr int LPR = D_PAD / VEC;        // lanes per K/V row
  static constexpr int TPL = kWaveSize / LPR;    // slots per wave-load
  static_assert(LPR >= 1 && LPR <= 32 && BS % TPL == 0, "unsupported tile shape");
  static constexpr int NLB = BS / TPL;           // wave-loads per block (per K or V)
  static_assert(NLB % 2 == 0, "slots of a block are paired for P.V");
  static constexpr int NG = 4 / NLB > 1 ? 4 / NLB : 1;   // blocks per load group
  static constexpr int NW = NWAVES;             // waves per workgroup
};

// Online-softmax state of one lane: m[h] is shared by the whole wave
// (wave-uniform); l[h] and acc[h][.] are this lane's partial sums over the
// slots it saw.
template <int G, int VEC>
struct LaneState {
  float m[G], l[G], acc[G][VEC];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[h][e] = 0.0f;
    }
  }
};

// One wave's pass over its blocks b_first, b_first + STRIDE, ... (nwb of them,
// may be <= 0) of one (sequence, KV head): QK^T, online softmax and P.V into
// `st`.
// ph holds the raw table entries of the first group (TableRow::raw, read by
// the caller, clamped to the row); head_off addresses this lane's row and channel chunk of the
// KV head inside a block.
template <int DT, int D_PAD, int G, int BS, int STRIDE = kDecodeWaves>
__device__ __forceinline__ void wave_accumulate(
    const DecodeParams& p, const TableRow& bt_row, const int L, const int b_first, const int nwb,
    const int64_t head_off, const int row, const uint4 (&qv)[G],
    int (&ph)[DecodeShape<DT, D_PAD, BS>::NG],
    LaneState<G, DecodeShape<DT, D_PAD, BS>::VEC>& st, Stamps* stamps = nullptr) {
  using S = DecodeShape<DT, D_PAD, BS>;
  constexpr int kElt = S::kElt, VEC = S::VEC, LPR = S::LPR, TPL = S::TPL, NLB = S::NLB;
  constexpr int NG = S::NG;
  float(&m)[G] = st.m;
  float(&l)[G] = st.l;
  float(&acc)[G][VEC] = st.acc;

  // One group of NG blocks: pass 1 computes the scores of every slot of the
  // group, the group max moves the running max once, pass 2 adds the weights
  // and P.V.
  auto compute_group = [&](const int g0, const uint4 (&kr)[NG][NLB], const uint4 (&vr)[NG][NLB]) {
      // Pass 1: scores of every slot of the group (log2 units). Every block of
      // the group is computed, so the group has a single path; a block past
      // this wave's share gets a limit of 0, which masks all its slots (its
      // loads were skipped and its registers are never used unmasked).
      float sc[NG][NLB][G];
  #pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int lim = g0 + i < nwb ? L : 0;
        const int tok0 = (b_first + (g0 + i) * STRIDE) * BS + row;
  #pragma unroll
        for (int j = 0; j < NLB; ++j) {
          const bool tok_ok = tok0 + j * TPL < lim;
  #pragma unroll
          for (int h = 0; h < G; ++h) {
            const float dot = row_sum<LPR>(dot16<DT>(kr[i][j], qv[h], 0.0f));
            sc[i][j][h] = tok_ok ? dot * p.scale_log2 : -INFINITY;
          }
        }
      }
      // One online-softmax step per group: the wave-wide max of the group's
      // scores becomes the new reference; earlier sums are rescaled once.
  #pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = sc[0][0][h];
  #pragma unroll
        for (int i = 0; i < NG; ++i)
  #pragma unroll
          for (int j = 0; j < NLB; ++j) mx = fmaxf(mx, sc[i][j][h]);
        const float m_new = fmaxf(m[h], wave_max_rows<LPR>(mx));   // finite: block g0 is valid
        const float alpha = __builtin_amdgcn_exp2f(m[h] - m_new);   // 0 when m = -inf
        m[h] = m_new;
        l[h] *= alpha;
  #pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] *= alpha;
      }
      // Pass 2: weights and P.V.
  #pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int lim = g0 + i < nwb ? L : 0;
        const int tok0 = (b_first + (g0 + i) * STRIDE) * BS + row;
        float w[NLB][G];
  #pragma unroll
        for (int j = 0; j < NLB; ++j)
  #pragma unroll
          for (int h = 0; h < G; ++h) {
            w[j][h] = __builtin_amdgcn_exp2f(sc[i][j][h] - m[h]);   // 0 for masked slots
            if constexpr (DT == NP_F32) l[h] += w[j][h];            // 16-bit: in pv_pair
          }
        uint4 vv[NLB];
  #pragma unroll
        for (int j = 0; j < NLB; ++j) {
          const bool tok_ok = tok0 + j * TPL < lim;
          vv[j].x = tok_ok ? vr[i][j].x : 0u;
          vv[j].y = tok_ok ? vr[i][j].y : 0u;
          vv[j].z = tok_ok ? vr[i][j].z : 0u;
          vv[j].w = tok_ok ? vr[i][j].w : 0u;
        }
        if constexpr (DT == NP_F32) {
  #pragma unroll
          for (int j = 0; j < NLB; ++j) {
            float vf[VEC];
            unpack16<DT>(vv[j], vf);
  #pragma unroll
            for (int h = 0; h < G; ++h)
  #pragma unroll
              for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(w[j][h], vf[e], acc[h][e]);
          }
        } else {
  #pragma unroll
          for (int j = 0; j < NLB; j += 2)
            pv_pair<DT, G, VEC>(vv[j], vv[j + 1], w, j, j + 1, acc, l);
        }
      }
  };
  // In the pipeline (every_block) every block of a group is loaded, so a
  // group issues the same number of loads on every path. (A load skipped on
  // one path makes the compiler's counter wait before a group's use also
  // cover the next group's loads, which then no longer overlap this group's
  // compute.) Every lane then reads the first 16 bytes of the pool for a
  // block past this wave's share (one line, so the load costs one request),
  // and the block is masked like any slot past the history. A wave with a
  // single group has nothing to overlap and skips such blocks.
  auto load_group = [&](const int g0, uint4 (&kr)[NG][NLB], uint4 (&vr)[NG][NLB],
                        const bool every_block) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const bool real = g0 + i < nwb;
      if (every_block || real) {
        const int64_t base =
            real ? int64_t(bt_row.phys(ph[i], b_first + (g0 + i) * STRIDE)) * p.kv_s0 + head_off
                 : 0;
        const int64_t step = real ? int64_t(TPL) * p.kv_s1 : 0;
#pragma unroll
        for (int j = 0; j < NLB; ++j) {
          kr[i][j] = load16_stream(p.k, base + j * step, kElt);
          vr[i][j] = load16_stream(p.v, base + j * step, kElt);
        }
      }
    }
    // Table entries of the group after the one just issued.
    if (g0 + NG < nwb) {
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int b = b_first + (g0 + NG + i) * STRIDE;
        ph[i] = bt_row.raw(b < p.max_blocks ? b : p.max_blocks - 1);
      }
    }
  };

  // Software pipeline over the ngr groups with two register buffers: the
  // loads of group g + 1 are in flight while group g computes. No load is
  // issued conditionally between a group's loads and its use, so every wait
  // before a group's compute leaves the next group's loads in flight; past
  // the last group the loop issues one group of stand-in loads (never
  // computed) instead of skipping the loads.
  const int ngr = nwb > 0 ? (nwb + NG - 1) / NG : 0;
  uint4 ka[NG][NLB], va[NG][NLB], kb[NG][NLB], vb[NG][NLB];
  if (ngr == 1) {
    load_group(0, ka, va, false);
    if (stamps != nullptr) stamps->at(2);
    compute_group(0, ka, va);
  } else if (ngr > 1) {
    load_group(0, ka, va, true);
    for (int g = 0; g < ngr; g += 2) {
      load_group((g + 1) * NG, kb, vb, true);
      if (stamps != nullptr && g == 0) stamps->at(2);
      compute_group(g * NG, ka, va);
      if (g + 1 >= ngr) break;
      load_group((g + 2) * NG, ka, va, true);
      compute_group((g + 1) * NG, kb, vb);
    }
  }

}

// Workgroup merge of the waves' states. The workgroup serves HW KV heads;
// wave k holds a partial state of head k % HW. Rows of a wave share m, so
// their sums add directly; the waves of one head are weighted by
// 2^(m_wave - M). Then, for each output pair of channels (c, c + 1) of query
// head h of the workgroup's HW * G (c < head_dim), emit(h, c, t0, t1, M, l)
// with the unnormalised sums. One barrier, plus one before the LDS writes
// when the workgroup reuses the buffers (sync_before).
template <int DT, int D_PAD, int G, int BS, int HW, int NWAVES = kDecodeWaves, typename Emit>
__device__ __forceinline__ void wg_combine(const DecodeParams& p, const int wave, const int lane,
                                           const int row, const int ch0,
                                           const LaneState<G, DecodeShape<DT, D_PAD, BS>::VEC>& st,
                                           const bool sync_before, Emit&& emit) {
  using S = DecodeShape<DT, D_PAD, BS, NWAVES>;
  constexpr int VEC = S::VEC, LPR = S::LPR, TPL = S::TPL, NW = S::NW;
  const float(&m)[G] = st.m;
  const float(&l)[G] = st.l;
  const float(&acc)[G][VEC] = st.acc;
  if (sync_before) __syncthreads();
  // The per-wave row sums (TPL rows) are formed in registers where the row
  // count is 8 (16-bit types, d_pad 64): partner rows are one DPP step and two
  // lane-swap steps apart, and each swap step halves the values a lane holds
  // (the transposed reduction), so LDS carries one partial per wave instead of
  // one per row.
  constexpr bool kRowsInRegs = LPR == 8;
  constexpr int NRW = kRowsInRegs ? 1 : TPL;   // partials per wave in LDS
  __shared__ float red_acc[NW][NRW][G][D_PAD];
  __shared__ float red_l[NW][NRW][G];
  __shared__ float red_m[NW][G];
  if constexpr (kRowsInRegs) {
    constexpr int N = G * VEC;                   // a multiple of 4
    constexpr int NL = (G + 3) / 4 * 4;
    float v[N], lv[NL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[h * VEC + e] = acc[h][e];
#pragma unroll
    for (int h = 0; h < NL; ++h) lv[h] = h < G ? l[h] : 0.0f;
    float u[N / 4], ul[NL / 4];
    rows8_sum<N>(v, u);
    rows8_sum<NL>(lv, ul);
    // u[k] in 16-lane group r = lane / 16 holds value 4k + r of this lane's
    // channel chunk (lanes 8..15 of a group duplicate lanes 0..7).
    const int r = lane / 16;
    if ((lane & 8) == 0) {
#pragma unroll
      for (int k = 0; k < N / 4; ++k) {
        const int vi = 4 * k + r;
        red_acc[wave][0][vi / VEC][ch0 + vi % VEC] = u[k];
      }
      if (lane % 16 == 0) {
#pragma unroll
        for (int k = 0; k < NL / 4; ++k)
          if (4 * k + r < G) red_l[wave][0][4 * k + r] = ul[k];
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (lane == 0) red_m[wave][h] = m[h];
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < VEC; e += 4)
        *reinterpret_cast<float4*>(&red_acc[wave][row][h][ch0 + e]) =
            make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
      if (lane % LPR == 0) red_l[wave][row][h] = l[h];
      if (lane == 0) red_m[wave][h] = m[h];
    }
  }
  __syncthreads();

  // Two channels per thread.
  constexpr int WPH = NW / HW;   // waves per head
  for (int o = threadIdx.x; o < HW * G * D_PAD / 2; o += NW * kWaveSize) {
    const int hh = o / (G * D_PAD / 2);   // head of the workgroup's HW
    const int h = (o / (D_PAD / 2)) % G;
    const int c = 2 * (o % (D_PAD / 2));
    float mm = -INFINITY;
#pragma unroll
    for (int j = 0; j < WPH; ++j) mm = fmaxf(mm, red_m[hh + j * HW][h]);
    float t0 = 0.0f, t1 = 0.0f, ll = 0.0f;
#pragma unroll
    for (int j = 0; j < WPH; ++j) {
      const int w = hh + j * HW;
      const float ww = __builtin_amdgcn_exp2f(red_m[w][h] - mm);   // 0 for idle waves
      float a0 = 0.0f, a1 = 0.0f, lw = 0.0f;
#pragma unroll
      for (int rr = 0; rr < NRW; ++rr) {
        const float2 a = *reinterpret_cast<const float2*>(&red_acc[w][rr][h][c]);
        a0 += a.x;
        a1 += a.y;
        lw += red_l[w][rr][h];
      }
      t0 = fmaf(ww, a0, t0);
      t1 = fmaf(ww, a1, t1);
      ll = fmaf(ww, lw, ll);
    }
    if (c >= p.head_dim) continue;
    emit(hh * G + h, c, t0, t1, mm, ll);
  }
}

template <int DT, int D_PAD, int G, int BS, bool FUSED>
__global__ __launch_bounds__(kDecodeWaves * kWaveSize) void paged_decode_kernel(
    const DecodeParams p) {
  using S = DecodeShape<DT, D_PAD, BS>;
  constexpr int kElt = S::kElt, VEC = S::VEC, LPR = S::LPR, NG = S::NG, NW = S::NW;

  const int kvh = blockIdx.x % p.hkv;
  const int split = blockIdx.x / p.hkv;
  const int s = blockIdx.y;
  const int b0 = split * p.bps;
  Stamps stamps;
  stamps.at(0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int lane = threadIdx.x % kWaveSize;
  const int row = lane / LPR;
  const int ch0 = (lane % LPR) * VEC;
  const bool chan_ok = ch0 < p.head_dim;
  const TableRow bt_row = table_row(p.bt, p.bt_stride, s, p.max_blocks, p.bt_contig);

  // This wave's blocks are b0 + wave + i * NW. It takes them in groups of NG:
  // all K/V loads of a group are issued before any of its blocks is used, the
  // loads of the next group are issued before this group computes, and table
  // entries are read one group ahead of their loads.
  // The first group's entries and this head group's q are read before the
  // context length is known (table reads are clamped to the row, q reads to
  // the real channels), so these reads share one memory round trip.
  int ph[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int b = b0 + wave + i * NW;
    ph[i] = bt_row.raw(b < p.max_blocks ? b : p.max_blocks - 1);
  }
  // q chunks of the G heads of this group. Padded channels load the last
  // real chunk and are zeroed by a select, so every lane loads.
  const int q_ch = chan_ok ? ch0 : p.head_dim - VEC;
  uint4 qv[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 t = load16(p.q, int64_t(s) * p.q_s0 + int64_t(kvh * G + h) * p.q_s1 + q_ch, kElt);
    qv[h] = chan_ok ? t : make_uint4(0, 0, 0, 0);
  }
  const int L = p.lens[s];
  // The table entries are needed only past the exit test below; tying them to
  // this point keeps the compiler from moving their reads after it (which
  // would add a second round trip before the first K/V load).
#pragma unroll
  for (int i = 0; i < NG; ++i) asm volatile("" ::"s"(ph[i]));
  int nb = (L + BS - 1) / BS;
  // A device length outside [1, table capacity], or longer than the grid of
  // this plan covers (the plan was made for shorter host lengths), has no
  // correct result here: the head group's outputs are set to NaN (by split
  // 0, which every plan launches) instead of dropping the blocks past the
  // last split.
  if (L < 1 || L > p.max_blocks * BS || nb > p.max_splits * p.bps) {
    if (split == 0) fill_nan<DT>(p, s, kvh * G, G);
    return;
  }
  int splits = (nb + p.bps - 1) / p.bps;
  stamps.at(1);
#ifdef NP_TRACE
  int32_t* trec = p.trace ? p.trace + (int64_t(blockIdx.y) * gridDim.x + blockIdx.x) *
                                          NP_TRACE_UNIFORM_WORDS
                          : nullptr;
  int32_t tflags = 1, tticket = -1;
  auto trace_write = [&]() {
    stamps.at(8);
    if (threadIdx.x != 0 || trec == nullptr) return;
    trec[0] = tflags;
    trec[1] = trace_where();
    trec[2] = s;
    trec[3] = kvh;
    trec[4] = split;
    trec[5] = b0;
    trec[6] = (b0 + p.bps) < nb ? (b0 + p.bps) : nb;
    trec[7] = tticket;
    trec[8] = splits;
    trec[9] = 0;
    for (int i = 0; i < kTraceStamps; ++i) {
      trec[10 + 2 * i] = int32_t(uint32_t(stamps.t[i]));
      trec[11 + 2 * i] = int32_t(uint32_t(stamps.t[i] >> 32));
    }
  };
  if (split >= splits) {
    if (threadIdx.x == 0 && trec != nullptr) trec[0] = 1;
    return;
  }
#else
  if (split >= splits) return;
#endif
  const int b1 = (b0 + p.bps) < nb ? (b0 + p.bps) : nb;
  const int nwb = (b1 - b0 - wave + NW - 1) / NW;   // blocks of this wave (may be <= 0)

  LaneState<G, VEC> st;
  st.reset();

  // Loads are unconditional inside a valid block: slots past the history are
  // still inside the block, and padded channels read the last real chunk
  // instead; both are masked by selects below, never by multiplication.
  const int64_t head_off = int64_t(kvh) * p.kv_s2 + q_ch + int64_t(row) * p.kv_s1;

  wave_accumulate<DT, D_PAD, G, BS>(p, bt_row, L, b0 + wave, nwb, head_off, row, qv, ph, st,
                                    &stamps);
  stamps.at(3);

  const bool direct = splits == 1;
  wg_combine<DT, D_PAD, G, BS, 1>(
      p, wave, lane, row, ch0, st, false,
      [&](int h, int c, float t0, float t1, float mm, float ll) {
        const int hg = kvh * G + h;
        if (direct) {
          const float r = __builtin_amdgcn_rcpf(ll);
          const int64_t oi = int64_t(s) * p.o_s0 + int64_t(hg) * p.o_s1 + c;
          store_out2<DT>(p.out, oi, t0 * r, t1 * r);
        } else {
          const int64_t part = (int64_t(s) * p.hq + hg) * p.max_splits + split;
          publish2(p.ws_acc + part * D_PAD + c, t0, t1);
          if (c == 0) publish2(p.ws_ml + 2 * part, mm, ll);
        }
      });
  stamps.at(4);
#ifdef NP_TRACE
  if (direct) tflags |= 4;
  if (!FUSED || direct) {
    trace_write();
    return;
  }
#endif
  if constexpr (FUSED) {
    if (direct) return;
    // Last-arriver merge: every thread waits until its partial stores are
    // complete, then one thread takes a ticket; the workgroup holding the last
    // ticket of its (sequence, KV head) merges all splits and resets the
    // counter for the next call. Counters sit kCounterStride apart so tickets
    // of different KV heads do not contend for one line.
    __shared__ int last;
    uint32_t* cnt = p.ws_cnt + int64_t(s * p.hkv + kvh) * kCounterStride;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    stamps.at(5);
    if (threadIdx.x == 0) {
      const uint32_t prev =
          __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = prev == uint32_t(splits - 1);
#ifdef NP_TRACE
      tticket = int32_t(prev);
#endif
    }
    __syncthreads();
    stamps.at(6);
    // Every workgroup runs the merge code, the others on a one-split dummy
    // that stores nothing. There is one call site, so one copy of the code:
    // the merging workgroup is the only one of its (sequence, KV head) on its
    // XCC that needs it, and its instruction fetches then find the lines in
    // the XCC's L2 instead of memory (measured: 0.2 us of the 4096-token
    // step).
    const bool is_last = last;
    merge_splits<DT, D_PAD, G>(p, s, kvh, is_last ? splits : 1, is_last);
#ifdef NP_TRACE
    if (!is_last) {
      trace_write();
      return;
    }
    tflags |= 2;
#else
    if (!is_last) return;
#endif
    if (threadIdx.x == 0)
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stamps.at(7);
#ifdef NP_TRACE
    trace_write();
#endif
  }
}

// ------------------------------------------------------ stream-K schedule
//
// For ragged batches. A workgroup serves HW KV heads at once (HW = 8, 4, 2 or
// 1, the largest that divides Hkv): its wave k takes head k % HW, and the
// NW / HW waves of one head take alternate blocks. So the HW heads of a block
// (8 x 128 contiguous bytes per slot for 16-bit d = 64 and 8 KV heads) are
// fetched by one workgroup at about the same time, rather than a head at a
// time by separate workgroups far apart in the launch; a read probe over the
// batching pool streams 4-head runs about 15% faster than single heads, and
// the kernel runs about 3% faster with 8 heads per workgroup than with 4.
//
// Every (sequence, head group) is a segment of nb_s block units followed by
// sk_cost virtual units that stand for the fixed cost of a segment (its q
// loads, pipeline fill and drain, combine and merge). The segments are laid
// end to end in (sequence, head group) order, U units in all, and workgroup w
// of the W in the launch takes units [w C, (w + 1) C) with C = ceil(U / W):
// every workgroup gets the same amount of work whatever the lengths, so no
// long split is left running alone at the end of the launch. The blocks of a
// segment that fall in one workgroup's range form a piece; a workgroup whose
// range holds only a segment's virtual units skips it. A segment with one
// piece writes its output directly; otherwise each piece publishes a partial
// and the last to arrive merges them. A workgroup can share only its first
// and its last piece with other workgroups, so a piece is stored in slot
// 2 w + side, side 0 if it starts at the workgroup's first unit and 1
// otherwise. The scan of the lengths runs on the device from context_lens, so
// the schedule always matches the lengths the kernel reads and the workspace
// bounds depend only on W.

// Merge of the n pieces of one segment, GG query heads from head0: every
// thread owns float4 chunks of the GG x d_pad output and folds in all pieces
// (UB loads in flight at a time), with the split-KV page's log-sum-exp
// weights as in merge_splits. No LDS, no barrier.
template <int DT, int D_PAD, int GG, int NWAVES, typename SlotOf>
__device__ __forceinline__ void merge_pieces(const DecodeParams& p, int s, int head0, int n,
                                             SlotOf&& slot_of) {
  constexpr int NCH = GG * D_PAD / 4;
  constexpr int UB = 4;
  n = __builtin_amdgcn_readfirstlane(n);
  // Piece j of head h is part slot_of(j) * GG + h. As in merge_splits, the
  // slot (the same for every lane) is a scalar offset of a buffer load over
  // the partial slots of the launch, 2 per workgroup; a lane's offset in a
  // slot is computed once.
  const __amdgpu_buffer_rsrc_t r_acc = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<void*>(p.ws_acc), 0, 2 * int(gridDim.x) * GG * D_PAD * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t r_ml = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<void*>(p.ws_ml), 0, 2 * int(gridDim.x) * GG * 8, kBufferWord3);
  // As in merge_splits, when a batch's (m, l) pairs fit one wave (UB * GG <=
  // 64), lane u * GG + h loads piece u's pair of head h once and the lanes
  // read theirs from the wave's LDS row; otherwise every lane loads its own.
  constexpr bool kShareMl = UB * GG <= kWaveSize;
  __shared__ float2 s_mlp[NWAVES][kWaveSize];
  const int wv = threadIdx.x / kWaveSize, ln = threadIdx.x % kWaveSize;
  const int pl = ln < UB * GG ? ln : UB * GG - 1;
  const int pu = pl / GG, phd = pl % GG;
  for (int chunk = threadIdx.x; chunk < NCH; chunk += NWAVES * kWaveSize) {
    const int h = (chunk * 4) / D_PAD;
    const int c = (chunk * 4) % D_PAD;
    const int acc_off = (h * D_PAD + c) * 4;
    const int ml_off = h * 8;
    float mx = -INFINITY, d = 0.0f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < n; j0 += UB) {
      float2 ml[UB];
      float4 a[UB];
      // Pieces past the last re-read the last one and get weight 0, so the
      // batch is issued without branches and consumed on every path (as in
      // merge_splits).
      u32x2_t mp = {0u, 0u};
      if constexpr (kShareMl)
        mp = __builtin_amdgcn_raw_buffer_load_b64(
            r_ml, (slot_of(j0 + pu < n ? j0 + pu : n - 1) * GG + phd) * 8, 0, kDeviceScopeLoad);
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int slot = __builtin_amdgcn_readfirstlane(slot_of(j0 + u < n ? j0 + u : n - 1));
        if constexpr (!kShareMl) {
          const u32x2_t m2 = __builtin_amdgcn_raw_buffer_load_b64(r_ml, ml_off, slot * GG * 8,
                                                                   kDeviceScopeLoad);
          ml[u] = make_float2(__uint_as_float(m2.x), __uint_as_float(m2.y));
        }
        const u32x4_t a4 = __builtin_amdgcn_raw_buffer_load_b128(
            r_acc, acc_off, slot * GG * D_PAD * 4, kDeviceScopeLoad);
        a[u] = make_float4(__uint_as_float(a4.x), __uint_as_float(a4.y), __uint_as_float(a4.z),
                           __uint_as_float(a4.w));
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kShareMl) {
        s_mlp[wv][ln] = make_float2(__uint_as_float(mp.x), __uint_as_float(mp.y));
#pragma unroll
        for (int u = 0; u < UB; ++u) ml[u] = s_mlp[wv][u * GG + h];
      }
#pragma unroll
      for (int u = 0; u < UB; ++u)
        if (j0 + u >= n) ml[u].x = -INFINITY;
      float m_new = mx;
#pragma unroll
      for (int u = 0; u < UB; ++u) m_new = fmaxf(m_new, ml[u].x);
      const float ms = m_new == -INFINITY ? 0.0f : m_new;
      const float aw = __builtin_amdgcn_exp2f(mx - ms);
      d *= aw;
      acc = make_float4(acc.x * aw, acc.y * aw, acc.z * aw, acc.w * aw);
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const float wu = __builtin_amdgcn_exp2f(ml[u].x - ms);
        d = fmaf(wu, ml[u].y, d);
        acc.x = fmaf(wu, a[u].x, acc.x);
        acc.y = fmaf(wu, a[u].y, acc.y);
        acc.z = fmaf(wu, a[u].z, acc.z);
        acc.w = fmaf(wu, a[u].w, acc.w);
      }
      mx = m_new;
    }
    const int64_t o = int64_t(s) * p.o_s0 + int64_t(head0 + h) * p.o_s1 + c;
    const float r = __builtin_amdgcn_rcpf(d);
    if (c < p.head_dim)
      store_out4<DT>(p.out, o, make_float4(acc.x * r, acc.y * r, acc.z * r, acc.w * r));
  }
}

// The 8-wave workgroup (launch bounds) allows up to 256 VGPRs per lane, two
// waves per SIMD: the planner's default of one workgroup per CU.
template <int DT, int D_PAD, int G, int BS, int HW>
__global__ __launch_bounds__(kSkWaves * kWaveSize) void paged_decode_sk_kernel(
    const DecodeParams p) {
  using S = DecodeShape<DT, D_PAD, BS, kSkWaves>;
  constexpr int kElt = S::kElt, VEC = S::VEC, LPR = S::LPR, NG = S::NG, NW = S::NW;
  constexpr int WPH = NW / HW;              // waves per head
  static_assert(NW % HW == 0, "heads per workgroup must divide the waves");
  __shared__ int sk_pre[kSkMaxSeqs + 1];    // units before each sequence's segments
  __shared__ int sk_last;
#ifdef NP_TRACE
  static_assert(NP_TRACE_SK_STAMP0 + NP_TRACE_SK_STAMP_WORDS <= NP_TRACE_SK_WORDS, "trace record");
  const uint64_t t_entry = __builtin_amdgcn_s_memrealtime();
#endif

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int w = blockIdx.x;
  const int W = gridDim.x;
  const int n_hg = p.hkv / HW;              // head groups: segments per sequence

  // Inclusive prefix sums of the per-sequence units, one wave, 64 sequences
  // per pass.
  if (wave == 0) {
    const int lane = threadIdx.x % kWaveSize;
    int carry = 0;
    for (int base = 0; base < p.num_seqs; base += kWaveSize) {
      const int s = base + lane;
      int u = 0;
      if (s < p.num_seqs) {
        int nb = (p.lens[s] + BS - 1) / BS;
        nb = nb < p.max_blocks ? nb : p.max_blocks;
        nb = nb > 0 ? nb : 0;
        u = (nb + p.sk_cost) * n_hg;
      }
#pragma unroll
      for (int d = 1; d < kWaveSize; d <<= 1) {
        const int t = __shfl_up(u, d);
        if (lane >= d) u += t;
      }
      if (s < p.num_seqs) sk_pre[s + 1] = carry + u;
      carry += __shfl(u, kWaveSize - 1);
    }
    if (lane == 0) sk_pre[0] = 0;
  }
  __syncthreads();
  // Values read from LDS are uniform across the workgroup; readfirstlane
  // tells the compiler so, which keeps the schedule in scalar registers and
  // its branches uniform.
  auto pre = [&](int i) { return __builtin_amdgcn_readfirstlane(sk_pre[i]); };
  const int U = pre(p.num_seqs);
  const int C = (U + W - 1) / W;
  int u = w * C;
  const int u_end = U < u + C ? U : u + C;
#ifdef NP_TRACE
  int32_t* trec = p.trace ? p.trace + int64_t(blockIdx.x) * NP_TRACE_SK_WORDS : nullptr;
  int32_t t_pieces = 0, t_overflow = 0;
  auto trace_header = [&](int n_merges) {
    if (threadIdx.x != 0 || trec == nullptr) return;
    trec[0] = t_pieces < NP_TRACE_SK_PIECES ? t_pieces : NP_TRACE_SK_PIECES;
    trec[1] = n_merges;
    trec[2] = trace_where();
    trec[3] = t_overflow;
    trec[4] = U;
    trec[5] = C;
    trec[6] = trec[7] = 0;
  };
  // Timestamp at word `at` of the stamp area (wave 0 waits for its memory
  // operations first; the other waves run on).
  auto sk_stamp = [&](int at, uint64_t t = 0) {
    if (trec == nullptr || threadIdx.x >= kWaveSize) return;
    if (t == 0) {
      __builtin_amdgcn_s_waitcnt(0);
      t = __builtin_amdgcn_s_memrealtime();
    }
    if (threadIdx.x == 0) {
      trec[NP_TRACE_SK_STAMP0 + at] = int32_t(uint32_t(t));
      trec[NP_TRACE_SK_STAMP0 + at + 1] = int32_t(uint32_t(t >> 32));
    }
  };
  sk_stamp(0, t_entry);
  sk_stamp(2);
  if (u >= u_end) {
    trace_header(0);
    sk_stamp(6);
    return;
  }
#else
  if (u >= u_end) return;
#endif
  // The sequence whose segments hold unit u: the last s with sk_pre[s] <= u
  // (every sequence has at least n_hg * sk_cost >= 1 units).
  int s = 0;
  {
    int hi = p.num_seqs - 1;
    while (s < hi) {
      const int mid = (s + hi + 1) / 2;
      if (pre(mid) <= u) s = mid;
      else hi = mid - 1;
    }
  }

  // Segments this workgroup has to merge (it held their last ticket). Only
  // its first and its last piece can be shared, so there are at most two;
  // the merges run after the loop, which keeps their registers out of it.
  int n_merge = 0;
  int mg_s[2] = {0, 0}, mg_hg[2] = {0, 0}, mg_n[2] = {0, 0}, mg_start[2] = {0, 0};
  bool first_piece = true;
  while (u < u_end) {
    if (u >= pre(s + 1)) ++s;   // u never passes a segment end, so one step
    const int L = ((ConstI32Ptr)p.lens)[s];   // scalar load (lengths are read-only)
    int nb = (L + BS - 1) / BS;
    nb = nb < p.max_blocks ? nb : p.max_blocks;
    nb = nb > 0 ? nb : 0;
    const int seg_units = nb + p.sk_cost;
    const int seq_start = pre(s);
    const int hg = (u - seq_start) / seg_units;
    const int seg_start = seq_start + hg * seg_units;
    const int seg_end = seg_start + seg_units;
    // Units that make pieces: the real blocks, or the first unit of a segment
    // without blocks (which then still writes its output).
    const int real_end = seg_start + (nb > 0 ? nb : 1);
    if (u >= real_end) {   // only virtual units of this segment here
      u = seg_end < u_end ? seg_end : u_end;
      continue;
    }
#ifdef NP_TRACE
    if (t_pieces < NP_TRACE_SK_PIECES) sk_stamp(8 + 4 * t_pieces);
#endif
    // Lane coordinates are derived afresh in every piece (from an opaque copy
    // of the thread index) so the compiler does not hoist lane-dependent
    // addresses out of the loop and keep them live across it.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid % kWaveSize;
    const int row = lane / LPR;
    const int ch0 = (lane % LPR) * VEC;
    const bool chan_ok = ch0 < p.head_dim;
    const int q_ch = chan_ok ? ch0 : p.head_dim - VEC;
    const int b_lo = u - seg_start;
    const int piece_end = u_end < real_end ? u_end : real_end;
    const int b_hi = (piece_end - seg_start) < nb ? (piece_end - seg_start) : nb;
    const int w_first = seg_start / C;
    const int n_pieces = (real_end - 1) / C - w_first + 1;
    const TableRow bt_row = table_row(p.bt, p.bt_stride, s, p.max_blocks, p.bt_contig);
    const int kvh = hg * HW + wave % HW;      // this wave's head
    const int phase = wave / HW;              // and its first block
    const int b_first = b_lo + phase;

    int ph[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int b = b_first + i * WPH;
      ph[i] = bt_row.raw(b < p.max_blocks ? b : p.max_blocks - 1);
    }
    uint4 qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 t =
          load16(p.q, int64_t(s) * p.q_s0 + int64_t(kvh * G + h) * p.q_s1 + q_ch, kElt);
      qv[h] = chan_ok ? t : make_uint4(0, 0, 0, 0);
    }
    const int nwb = (b_hi - b_first + WPH - 1) / WPH;   // blocks of this wave (may be <= 0)
    LaneState<G, VEC> st;
    st.reset();
    const int64_t head_off = int64_t(kvh) * p.kv_s2 + q_ch + int64_t(row) * p.kv_s1;
    wave_accumulate<DT, D_PAD, G, BS, WPH>(p, bt_row, L, b_first, nwb, head_off, row, qv, ph,
                                           st);

    const bool direct = n_pieces == 1;
    const int slot = 2 * w + (u == w * C ? 0 : 1);
    const int head0 = hg * HW * G;            // first query head of the segment
    wg_combine<DT, D_PAD, G, BS, HW, kSkWaves>(
        p, wave, lane, row, ch0, st, !first_piece,
        [&](int h, int c, float t0, float t1, float mm, float ll) {
          if (direct) {
            const float r = __builtin_amdgcn_rcpf(ll);
            const int64_t oi = int64_t(s) * p.o_s0 + int64_t(head0 + h) * p.o_s1 + c;
            store_out2<DT>(p.out, oi, t0 * r, t1 * r);
          } else {
            const int64_t part = int64_t(slot) * (HW * G) + h;
            publish2(p.ws_acc + part * D_PAD + c, t0, t1);
            if (c == 0) publish2(p.ws_ml + 2 * part, mm, ll);
          }
        });
    first_piece = false;
#ifdef NP_TRACE
    const bool t_keep = trec != nullptr && t_pieces < NP_TRACE_SK_PIECES;
    int32_t* tp = t_keep ? trec + 8 + 8 * t_pieces : nullptr;
    if (t_pieces >= NP_TRACE_SK_PIECES) t_overflow = 1;
    if (threadIdx.x == 0 && t_keep) {
      tp[0] = s;
      tp[1] = hg;
      tp[2] = b_lo;
      tp[3] = b_hi;
      tp[4] = direct ? -1 : slot;
      tp[5] = n_pieces;
      tp[6] = -1;
      tp[7] = u;
    }
#endif
    if (!direct) {
      // Ticket, with the ordering of the split kernel's: stores complete,
      // then the ticket.
      uint32_t* cnt = p.ws_cnt + int64_t(s * p.hkv + hg) * kCounterStride;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sk_last = prev == uint32_t(n_pieces - 1);
#ifdef NP_TRACE
        if (t_keep) tp[6] = int32_t(prev);
#endif
      }
      __syncthreads();
      if (__builtin_amdgcn_readfirstlane(sk_last)) {
        const int i = n_merge++ > 0 ? 1 : 0;
        mg_s[i] = s;
        mg_hg[i] = hg;
        mg_n[i] = n_pieces;
        mg_start[i] = seg_start;
      }
    }
#ifdef NP_TRACE
    if (t_pieces < NP_TRACE_SK_PIECES) sk_stamp(10 + 4 * t_pieces);
    ++t_pieces;
#endif
    u = seg_end < u_end ? seg_end : u_end;
  }
#ifdef NP_TRACE
  sk_stamp(4);
#endif
  for (int i = 0; i < n_merge; ++i) {
    const int ms = i ? mg_s[1] : mg_s[0];
    const int mh = i ? mg_hg[1] : mg_hg[0];
    const int mn = i ? mg_n[1] : mg_n[0];
    const int m0 = i ? mg_start[1] : mg_start[0];
    const int wf = m0 / C;
    // Piece j belongs to workgroup wf + j; only the first can start inside
    // its workgroup's range.
    auto slot_of = [&](int j) {
      const int wj = wf + j;
      const int side = (j == 0 && m0 != wj * C) ? 1 : 0;
      return 2 * wj + side;
    };
#ifdef NP_TRACE
    if (threadIdx.x == 0 && trec != nullptr) {
      int32_t* tm = trec + NP_TRACE_SK_MERGE0 + NP_TRACE_SK_MERGE_WORDS * i;
      tm[0] = ms;
      tm[1] = mh;
      tm[2] = mn;
      tm[3] = m0;
      tm[4] = wf;
      tm[5] = tm[6] = tm[7] = 0;
      for (int j = 0; j < mn && j < NP_TRACE_SK_SLOTS; ++j) tm[8 + j] = slot_of(j);
      if (mn > NP_TRACE_SK_SLOTS) t_overflow = 1;
    }
#endif
#ifdef NP_TRACE
    sk_stamp(8 + 4 * NP_TRACE_SK_PIECES + 4 * i);
#endif
    merge_pieces<DT, D_PAD, HW * G, kSkWaves>(p, ms, mh * HW * G, mn, slot_of);
#ifdef NP_TRACE
    sk_stamp(10 + 4 * NP_TRACE_SK_PIECES + 4 * i);
#endif
    // The next call that uses the counter is ordered after this launch.
    if (threadIdx.x == 0)
      __hip_atomic_store(p.ws_cnt + int64_t(ms * p.hkv + mh) * kCounterStride, 0u,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#ifdef NP_TRACE
  trace_header(n_merge);
  sk_stamp(6);
#endif
}

// Separate-launch merge of every (sequence, KV head) that was split.
template <int DT, int D_PAD, int G, int BS>
__global__ __launch_bounds__(256) void split_combine_kernel(const DecodeParams p) {
  const int kvh = blockIdx.x % p.hkv;
  const int s = blockIdx.x / p.hkv;
  const int L = p.lens[s];
  const int nb = (L + BS - 1) / BS;
  // Lengths the decode kernel rejected (their outputs hold NaN) are left alone.
  if (L < 1 || L > p.max_blocks * BS || nb > p.max_splits * p.bps) return;
  const int splits = (nb + p.bps - 1) / p.bps;
  if (splits <= 1) return;
  merge_splits<DT, D_PAD, G>(p, s, kvh, splits);
}

template <int DT, int D_PAD, int G>
np_status launch_decode_t(const DecodeParams& prm, const np_plan_core& c, hipStream_t st) {
  constexpr int BS = 16;
  dim3 grid(c.grid[0], c.grid[1], c.grid[2]);
  if (c.schedule == kScheduleStreamK) {
    switch (sk_heads_per_wg(c.hkv)) {
      case 8: paged_decode_sk_kernel<DT, D_PAD, G, BS, 8><<<grid, dim3(c.wg_size), 0, st>>>(prm); break;
      case 4: paged_decode_sk_kernel<DT, D_PAD, G, BS, 4><<<grid, dim3(c.wg_size), 0, st>>>(prm); break;
      case 2: paged_decode_sk_kernel<DT, D_PAD, G, BS, 2><<<grid, dim3(c.wg_size), 0, st>>>(prm); break;
      default: paged_decode_sk_kernel<DT, D_PAD, G, BS, 1><<<grid, dim3(c.wg_size), 0, st>>>(prm); break;
    }
    return hipGetLastError() == hipSuccess ? NP_OK : NP_ERR_HIP;
  }
  if (c.fused_combine)
    paged_decode_kernel<DT, D_PAD, G, BS, true><<<grid, dim3(c.wg_size), 0, st>>>(prm);
  else
    paged_decode_kernel<DT, D_PAD, G, BS, false><<<grid, dim3(c.wg_size), 0, st>>>(prm);
  if (hipGetLastError() != hipSuccess) return NP_ERR_HIP;
  if (c.combine_wgs) {
    split_combine_kernel<DT, D_PAD, G, BS><<<dim3(c.combine_wgs), dim3(256), 0, st>>>(prm);
    if (hipGetLastError() != hipSuccess) return NP_ERR_HIP;
  }
  return NP_OK;
}

template <int DT, int D_PAD>
np_status launch_decode_g(const DecodeParams& prm, const np_plan_core& c, hipStream_t st) {
  switch (c.group) {
    case 1: return launch_decode_t<DT, D_PAD, 1>(prm, c, st);
    case 2: return launch_decode_t<DT, D_PAD, 2>(prm, c, st);
    case 3: return launch_decode_t<DT, D_PAD, 3>(prm, c, st);
    case 4: return launch_decode_t<DT, D_PAD, 4>(prm, c, st);
    case 5: return launch_decode_t<DT, D_PAD, 5>(prm, c, st);
    case 6: return launch_decode_t<DT, D_PAD, 6>(prm, c, st);
    case 7: return launch_decode_t<DT, D_PAD, 7>(prm, c, st);
    case 8: return launch_decode_t<DT, D_PAD, 8>(prm, c, st);
    default: return NP_ERR_UNSUPPORTED;
  }
}

template <int DT>
np_status launch_decode_d(const DecodeParams& prm, const np_plan_core& c, hipStream_t st) {
  switch (c.d_pad) {
    case 64: return launch_decode_g<DT, 64>(prm, c, st);
    case 128: return launch_decode_g<DT, 128>(prm, c, st);
    default: return NP_ERR_UNSUPPORTED;
  }
}

}  // namespace

}  // namespace np

using namespace np;

namespace {
np_status decode_call(const np_paged_desc* desc, const np_plan_t* plan, const void* q,
                      const void* k_pool, const void* v_pool, const int32_t* block_table,
                      const int32_t* context_lens, void* out, void* workspace,
                      size_t workspace_bytes, void* stream);
}  // namespace

#ifdef NP_TRACE
namespace {
void* g_trace = nullptr;
size_t g_trace_bytes = 0;
}  // namespace

extern "C" np_status np_debug_set_trace(void* buf, size_t bytes) {
  if (buf != nullptr && reinterpret_cast<uintptr_t>(buf) % 4 != 0) return NP_ERR_MISALIGNED;
  g_trace = buf;
  g_trace_bytes = buf ? bytes : 0;
  return NP_OK;
}
#endif

extern "C" np_status np_paged_attention_decode(const np_paged_desc* desc,
                                               const np_plan_t* plan, const void* q,
                                               const void* k_pool, const void* v_pool,
                                               const int32_t* block_table,
                                               const int32_t* context_lens, void* out,
                                               void* workspace, size_t workspace_bytes,
                                               void* stream) {
  return decode_call(desc, plan, q, k_pool, v_pool, block_table, context_lens, out, workspace,
                     workspace_bytes, stream);
}

namespace {

// ------------------------------------------------- allocation-free variant
//
// For callers that cannot allocate (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc): the decode workspace is this
// file-scope device array instead of a caller buffer. Each GPU the library
// runs on holds its own copy until the process ends. In host code `scratch`
// names a host-side stand-in, not device memory: its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever passed to kernels.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ __launch_bounds__(256) void scratch_clear_kernel(uint4* p, size_t n16) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16;
       i += size_t(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// The current device's scratch address; on a device's first call, looks it
// up and clears the array on `stream` with a fill kernel (the arrival
// counters at its start must begin at zero; every decode call leaves them
// zero again).
np_status scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NP_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return NP_ERR_HIP;
    scratch_clear_kernel<<<dim3(1024), dim3(256), 0, stream>>>(static_cast<uint4*>(ptr),
                                                               kScratchBytes / 16);
    if (hipGetLastError() != hipSuccess) return NP_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return NP_OK;
}

}  // namespace

extern "C" np_status np_paged_attention_decode_noalloc(const np_paged_desc* desc,
                                                       const np_plan_t* plan, const void* q,
                                                       const void* k_pool, const void* v_pool,
                                                       const int32_t* block_table,
                                                       const int32_t* context_lens, void* out,
                                                       void* stream) {
  np_status st = check_desc(desc);
  if (st != NP_OK) return st;
  st = check_pointers(desc, q, k_pool, v_pool, block_table, context_lens, out);
  if (st != NP_OK) return st;
  st = check_plan(desc, plan, 0);
  if (st != NP_OK) return st;
  if (plan->core.ws_bytes > kScratchBytes) return NP_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  st = scratch_for_current_device(static_cast<hipStream_t>(stream), &ws);
  if (st != NP_OK) return st;
  return decode_call(desc, plan, q, k_pool, v_pool, block_table, context_lens, out, ws,
                     kScratchBytes, stream);
}

namespace {

np_status decode_call(const np_paged_desc* desc, const np_plan_t* plan, const void* q,
                      const void* k_pool, const void* v_pool, const int32_t* block_table,
                      const int32_t* context_lens, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  np_status st = check_desc(desc);
  if (st != NP_OK) return st;
  st = check_pointers(desc, q, k_pool, v_pool, block_table, context_lens, out);
  if (st != NP_OK) return st;
  st = check_plan(desc, plan, 0);
  if (st != NP_OK) return st;
  const np_plan_core& c = plan->core;
  if (desc->n_q_total != desc->num_seqs) return NP_ERR_BAD_SHAPE;
  if (c.block_size != 16 || c.group > kMaxGroup || c.head_dim > 128 ||
      (c.d_pad != 64 && c.d_pad != 128))
    return NP_ERR_UNSUPPORTED;
  if (c.ws_bytes > 0) {
    if (workspace == nullptr) return NP_ERR_NULL_PTR;
    if (reinterpret_cast<uintptr_t>(workspace) % kWsAlign != 0) return NP_ERR_MISALIGNED;
    if (workspace_bytes < c.ws_bytes) return NP_ERR_WORKSPACE_TOO_SMALL;
  }
  DecodeParams prm{};
  prm.q = q;
  prm.k = k_pool;
  prm.v = v_pool;
  // A NULL table (contiguous layout) reads a stand-in row: see np_table.h.
  prm.bt = block_table ? block_table : context_lens;
  prm.bt_contig = block_table == nullptr;
  prm.lens = context_lens;
  prm.out = out;
  prm.ws_cnt = c.ws_bytes
                   ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + c.ws_cnt_off)
                   : nullptr;
  prm.ws_ml = c.ws_bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) + c.ws_ml_off)
                         : nullptr;
  prm.ws_acc = c.ws_bytes
                   ? reinterpret_cast<float*>(static_cast<char*>(workspace) + c.ws_acc_off)
                   : nullptr;
  prm.q_s0 = desc->q_stride[0];
  prm.q_s1 = desc->q_stride[1];
  prm.kv_s0 = desc->kv_stride[0];
  prm.kv_s1 = desc->kv_stride[1];
  prm.kv_s2 = desc->kv_stride[2];
  prm.o_s0 = desc->out_stride[0];
  prm.o_s1 = desc->out_stride[1];
  prm.bt_stride = block_table ? desc->bt_stride : 0;
  prm.hkv = c.hkv;
  prm.hq = c.hq;
  prm.head_dim = c.head_dim;
  prm.max_blocks = c.max_blocks;
  prm.bps = c.blocks_per_split;
  prm.max_splits = c.max_splits;
  prm.num_seqs = c.num_seqs;
  prm.sk_cost = c.sk_cost;
  const float scale = desc->scale > 0.0f ? desc->scale : 1.0f / std::sqrt(float(c.head_dim));
  prm.scale_log2 = scale * kLog2e;
  prm.trace = nullptr;
#ifdef NP_TRACE
  if (g_trace != nullptr) {
    const size_t words = c.schedule == kScheduleStreamK ? NP_TRACE_SK_WORDS
                                                        : NP_TRACE_UNIFORM_WORDS;
    const size_t need = size_t(c.grid[0]) * c.grid[1] * c.grid[2] * words * sizeof(int32_t);
    if (g_trace_bytes < need) return NP_ERR_WORKSPACE_TOO_SMALL;
    prm.trace = static_cast<int32_t*>(g_trace);
  }
#endif
  hipStream_t hs = static_cast<hipStream_t>(stream);
  switch (c.dtype) {
    case NP_F32: return launch_decode_d<NP_F32>(prm, c, hs);
    case NP_F16: return launch_decode_d<NP_F16>(prm, c, hs);
    case NP_BF16: return launch_decode_d<NP_BF16>(prm, c, hs);
    default: return NP_ERR_BAD_DTYPE;
  }
}

}  // namespace
