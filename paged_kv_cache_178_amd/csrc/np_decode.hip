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
// * Waves take whole blocks round-robin and prefetch the next block's K/V into
//   registers while computing the current one.
// * Each group of LPR lanes ("row") runs its own online softmax over the slots
//   it sees ("What a Kernel Is ...", "Technical Details": running max and
//   sum). No cross-lane max is needed in the loop; the only cross-lane work is
//   the LPR-lane sum of the QK partial dot products (DPP).
// * The running max is only moved when a score exceeds it by more than
//   kLazy (log2 units), so the accumulator is rarely rescaled; weights stay
//   below 2^kLazy, which fp32 holds exactly as well as weights below 1.
// * At the end the rows and waves are merged through LDS.
// Scores are kept in log2 units (scale * log2 e folded in), exp2 is v_exp_f32.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "np_internal.h"

namespace np {

namespace {

constexpr float kLazy = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* bt;
  const int32_t* lens;
  void* out;
  float* ws_ml;
  float* ws_acc;
  int64_t q_s0, q_s1;
  int64_t kv_s0, kv_s1, kv_s2;
  int64_t o_s0, o_s1;
  int64_t bt_stride;
  int32_t hkv, hq, head_dim, max_blocks, bps, max_splits;
  float scale_log2;
};

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

// Unpack a 16-byte chunk into fp32 values (8 for 16-bit types, 4 for fp32).
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& a, float* f);

template <>
__device__ __forceinline__ void unpack16<NP_BF16>(const uint4& a, float* f) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void unpack16<NP_F16>(const uint4& a, float* f) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2_t h = __builtin_bit_cast(f16x2_t, w[i]);
    f[2 * i] = static_cast<float>(h.x);
    f[2 * i + 1] = static_cast<float>(h.y);
  }
}

template <>
__device__ __forceinline__ void unpack16<NP_F32>(const uint4& a, float* f) {
  f[0] = __uint_as_float(a.x);
  f[1] = __uint_as_float(a.y);
  f[2] = __uint_as_float(a.z);
  f[3] = __uint_as_float(a.w);
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

__device__ __forceinline__ uint4 load16(const void* base, int64_t elem_off, int elt) {
  return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + elem_off * elt);
}

// ------------------------------------------------------------------ kernel

template <int DT, int D_PAD, int G, int BS>
__global__ __launch_bounds__(kDecodeWaves * kWaveSize) void paged_decode_kernel(
    const DecodeParams p) {
  constexpr int kElt = Elt<DT>::kBytes;
  constexpr int VEC = 16 / kElt;          // elements per lane-load
  constexpr int LPR = D_PAD / VEC;        // lanes per K/V row
  constexpr int TPL = kWaveSize / LPR;    // slots per wave-load
  static_assert(LPR >= 1 && LPR <= 32 && BS % TPL == 0, "unsupported tile shape");
  constexpr int NLB = BS / TPL;           // wave-loads per block (per K or V)
  constexpr int NW = kDecodeWaves;

  const int kvh = blockIdx.x % p.hkv;
  const int split = blockIdx.x / p.hkv;
  const int s = blockIdx.y;
  const int L = p.lens[s];
  int nb = (L + BS - 1) / BS;
  nb = nb < p.max_blocks ? nb : p.max_blocks;
  const int splits = (nb + p.bps - 1) / p.bps;
  if (split >= splits) return;
  const int b0 = split * p.bps;
  const int b1 = (b0 + p.bps) < nb ? (b0 + p.bps) : nb;

  const int wave = threadIdx.x / kWaveSize;
  const int lane = threadIdx.x % kWaveSize;
  const int row = lane / LPR;
  const int ch0 = (lane % LPR) * VEC;
  const bool chan_ok = ch0 < p.head_dim;

  // q chunks of the G heads of this group (zero in padded channels).
  uint4 qv[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    qv[h] = make_uint4(0, 0, 0, 0);
    if (chan_ok)
      qv[h] = load16(p.q, int64_t(s) * p.q_s0 + int64_t(kvh * G + h) * p.q_s1 + ch0, kElt);
  }

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.0f;
  }

  const int32_t* bt_row = p.bt + int64_t(s) * p.bt_stride;
  const int64_t head_off = int64_t(kvh) * p.kv_s2 + ch0;

  uint4 kc[NLB], vc[NLB];
  auto issue = [&](int b, uint4* kk, uint4* vv) {
    const int64_t base = int64_t(bt_row[b]) * p.kv_s0 + head_off;
#pragma unroll
    for (int j = 0; j < NLB; ++j) {
      const int slot = j * TPL + row;
      const bool ok = chan_ok && (b * BS + slot < L);
      kk[j] = make_uint4(0, 0, 0, 0);
      vv[j] = make_uint4(0, 0, 0, 0);
      if (ok) {
        kk[j] = load16(p.k, base + int64_t(slot) * p.kv_s1, kElt);
        vv[j] = load16(p.v, base + int64_t(slot) * p.kv_s1, kElt);
      }
    }
  };

  int b = b0 + wave;
  if (b < b1) issue(b, kc, vc);
  for (; b < b1; b += NW) {
    uint4 kn[NLB], vn[NLB];
    const bool more = b + NW < b1;
    if (more) issue(b + NW, kn, vn);

    // Scores of this row's NLB slots for the G heads (log2 units).
    float sc[NLB][G];
#pragma unroll
    for (int j = 0; j < NLB; ++j) {
      const bool tok_ok = b * BS + j * TPL + row < L;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float dot = row_sum<LPR>(dot16<DT>(kc[j], qv[h], 0.0f));
        sc[j][h] = tok_ok ? dot * p.scale_log2 : -INFINITY;
      }
    }
    // Online softmax update, lazily moving the reference max.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = sc[0][h];
#pragma unroll
      for (int j = 1; j < NLB; ++j) mx = fmaxf(mx, sc[j][h]);
      if (mx > m[h] + kLazy) {
        const float alpha = __builtin_amdgcn_exp2f(m[h] - mx);   // 0 when m = -inf
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] *= alpha;
        m[h] = mx;
      }
    }
    float vf[NLB][VEC];
#pragma unroll
    for (int j = 0; j < NLB; ++j) unpack16<DT>(vc[j], vf[j]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      // m[h] is finite once the row has seen a valid slot; before that every
      // sc is -inf and the row's weights must stay 0.
      const float mref = m[h] == -INFINITY ? 0.0f : m[h];
#pragma unroll
      for (int j = 0; j < NLB; ++j) {
        const float w = __builtin_amdgcn_exp2f(sc[j][h] - mref);
        l[h] += w;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(w, vf[j][e], acc[h][e]);
      }
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < NLB; ++j) {
        kc[j] = kn[j];
        vc[j] = vn[j];
      }
    }
  }

  // ---- merge the NW x TPL row states of the workgroup through LDS.
  __shared__ float red_acc[NW][TPL][G][D_PAD];
  __shared__ float red_m[NW * TPL * G];
  __shared__ float red_l[NW * TPL * G];
  __shared__ float red_w[NW * TPL * G];
  __shared__ float fin_m[G];
  __shared__ float fin_l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) red_acc[wave][row][h][ch0 + e] = acc[h][e];
    if (lane % LPR == 0) {
      red_m[(wave * TPL + row) * G + h] = m[h];
      red_l[(wave * TPL + row) * G + h] = l[h];
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float mm = -INFINITY;
    for (int r = 0; r < NW * TPL; ++r) mm = fmaxf(mm, red_m[r * G + h]);
    float ll = 0.0f;
    for (int r = 0; r < NW * TPL; ++r) {
      const float w = __builtin_amdgcn_exp2f(red_m[r * G + h] - mm);   // 0 for empty rows
      red_w[r * G + h] = w;
      ll += w * red_l[r * G + h];
    }
    fin_m[h] = mm;
    fin_l[h] = ll;
  }
  __syncthreads();

  const bool direct = splits == 1;
  for (int o = threadIdx.x; o < G * D_PAD; o += NW * kWaveSize) {
    const int h = o / D_PAD;
    const int c = o % D_PAD;
    if (c >= p.head_dim) continue;
    float tot = 0.0f;
#pragma unroll
    for (int r = 0; r < NW * TPL; ++r)
      tot = fmaf(red_w[r * G + h], red_acc[r / TPL][r % TPL][h][c], tot);
    const int hg = kvh * G + h;
    if (direct) {
      store_out<DT>(p.out, int64_t(s) * p.o_s0 + int64_t(hg) * p.o_s1 + c, tot / fin_l[h]);
    } else {
      const int64_t part = (int64_t(s) * p.hq + hg) * p.max_splits + split;
      p.ws_acc[part * D_PAD + c] = tot;
      if (c == 0) {
        p.ws_ml[2 * part] = fin_m[h];
        p.ws_ml[2 * part + 1] = fin_l[h];
      }
    }
  }
}

// Merge the splits of every (sequence, KV head) that was split: with
// M = max_j m_j, out = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j. This
// is the split-KV page's log-sum-exp combine written with unnormalised
// partials (lse_j = m_j + log l_j, out_j = acc_j / l_j).
template <int DT, int D_PAD, int G, int BS>
__global__ __launch_bounds__(256) void split_combine_kernel(const DecodeParams p) {
  const int kvh = blockIdx.x % p.hkv;
  const int s = blockIdx.x / p.hkv;
  const int L = p.lens[s];
  int nb = (L + BS - 1) / BS;
  nb = nb < p.max_blocks ? nb : p.max_blocks;
  int splits = (nb + p.bps - 1) / p.bps;
  splits = splits < p.max_splits ? splits : p.max_splits;
  if (splits <= 1) return;
  for (int o = threadIdx.x; o < G * D_PAD; o += blockDim.x) {
    const int h = o / D_PAD;
    const int c = o % D_PAD;
    if (c >= p.head_dim) continue;
    const int hg = kvh * G + h;
    const int64_t part0 = (int64_t(s) * p.hq + hg) * p.max_splits;
    float mm = -INFINITY;
    for (int j = 0; j < splits; ++j) mm = fmaxf(mm, p.ws_ml[2 * (part0 + j)]);
    float num = 0.0f, den = 0.0f;
    for (int j = 0; j < splits; ++j) {
      const float w = __builtin_amdgcn_exp2f(p.ws_ml[2 * (part0 + j)] - mm);
      den = fmaf(w, p.ws_ml[2 * (part0 + j) + 1], den);
      num = fmaf(w, p.ws_acc[(part0 + j) * D_PAD + c], num);
    }
    store_out<DT>(p.out, int64_t(s) * p.o_s0 + int64_t(hg) * p.o_s1 + c, num / den);
  }
}

template <int DT, int D_PAD, int G>
np_status launch_decode_t(const DecodeParams& prm, const np_plan_core& c, hipStream_t st) {
  constexpr int BS = 16;
  dim3 grid(c.grid[0], c.grid[1], c.grid[2]);
  paged_decode_kernel<DT, D_PAD, G, BS><<<grid, dim3(c.wg_size), 0, st>>>(prm);
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

extern "C" np_status np_paged_attention_decode(const np_paged_desc* desc,
                                               const np_plan_t* plan, const void* q,
                                               const void* k_pool, const void* v_pool,
                                               const int32_t* block_table,
                                               const int32_t* context_lens, void* out,
                                               void* workspace, size_t workspace_bytes,
                                               void* stream) {
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
  prm.bt = block_table;
  prm.lens = context_lens;
  prm.out = out;
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
  prm.bt_stride = desc->bt_stride;
  prm.hkv = c.hkv;
  prm.hq = c.hq;
  prm.head_dim = c.head_dim;
  prm.max_blocks = c.max_blocks;
  prm.bps = c.blocks_per_split;
  prm.max_splits = c.max_splits;
  const float scale = desc->scale > 0.0f ? desc->scale : 1.0f / std::sqrt(float(c.head_dim));
  prm.scale_log2 = scale * kLog2e;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  switch (c.dtype) {
    case NP_F32: return launch_decode_d<NP_F32>(prm, c, hs);
    case NP_F16: return launch_decode_d<NP_F16>(prm, c, hs);
    case NP_BF16: return launch_decode_d<NP_BF16>(prm, c, hs);
    default: return NP_ERR_BAD_DTYPE;
  }
}
