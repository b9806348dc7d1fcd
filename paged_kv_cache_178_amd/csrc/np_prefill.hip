// Chunked prefill over a paged KV cache on the gfx950 matrix cores.
//
// What is computed ("I Wrote the Three Attention Kernels That Run LLM
// Inference -- in Portable Triton, on a Free Colab T4", sections "What is
// attention, really?", "1. Fused prefill attention" and "3. Paged KV-cache
// attention"; "Day 23: the real triton.jit paged-attention kernel", section
// "What I added today", for past): for query row i of sequence s (absolute
// position past_s + i) and query head h,
//   out[q_start[s]+i, h, :] = sum_{t <= past_s+i} softmax_t(scale <q, K_s[t]>) V_s[t]
// with K_s[t], V_s[t] read through the block table, KV head h / G.
//
// Decomposition:
// * One 512-thread workgroup (8 wave64) per (sequence, KV head, tile). A tile
//   is 4 units; a unit is one query head of the GQA group times 64 query rows
//   (units numbered head-fastest), so the waves of a workgroup share every
//   K/V tile they stage: for G = 4 the four heads of the group.
// * Each unit has two waves, one in each of two wave groups; group g takes key
//   tiles g, g + 2, g + 4, ..., and at the end group 1 hands its (m, l, acc)
//   to group 0 through LDS for the split-KV log-sum-exp merge. A wave holds
//   its 64 query rows as two 32-column MFMA blocks, so every K and V^T
//   operand read from LDS feeds two MFMAs.
// * Key tiles of 64 keys (4 blocks of 16) are staged in LDS in three buffers
//   per group, one tile per group per step, loaded two steps ahead straight
//   from global memory into LDS (no register staging): K and V both as
//   [key][channel] rows. Wave w loads block w % 4 of its group's tile. The
//   workgroup copies its sequence's table row to LDS once, so a step finds its
//   block without a scalar load from global memory.
// * S^T = K Q^T on v_mfma_f32_32x32x16 (A = K rows from LDS, B = 32 of the
//   wave's query rows held in registers), so each lane holds one query's scores:
//   the online-softmax max and sum ("1. Fused prefill attention": stream K/V,
//   reduce online, never materialise N x N) stay in the lane, plus one
//   exchange with the lane 32 away.
// * O^T += V^T P^T on the same MFMA: P^T stays in the registers it was
//   computed in (rounded to the input type); the keys of each k-step are taken
//   in the order those registers hold them, and the V^T operand is read in the
//   same order from the [key][channel] rows by a transposing LDS read.
// * Scores are in log2 units (scale * log2 e folded in); exp2 is v_exp_f32.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "np_internal.h"
#include "np_table.h"

namespace np {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;       // log2 units: weights stay below 256
constexpr int kKT = 64;             // keys per staged tile
constexpr int kD = 64;              // head_dim handled by this kernel
constexpr int kStages = 3;         // LDS tile buffers per wave group (loads run 2 steps ahead)
// Table entries a workgroup copies to LDS (longer histories read the rest
// from the table in global memory).
constexpr int kTabCache = 1024;

// K and V tiles sit in LDS as [key][channel] rows of 128 bytes, written straight
// from global memory (global_load_lds: lane l's 16 bytes land at base + 16 l)
// with the 16-byte chunks of each row permuted by an XOR swizzle, so that each
// 256-byte pass of an operand read touches every one of the 64 four-byte LDS
// banks once (two key rows share one span of the banks, the even key's row
// first):
// * K (MFMA A operand of S^T, 16-byte reads): a pass reads chunk c of 16
//   consecutive keys; slot c ^ ((key >> 1) & 7) gives the 8 even keys 8
//   distinct slots, and the 8 odd keys likewise.
// * V (ds_read_b64_tr_b16, 8-byte transposing reads): a pass reads chunks
//   c .. c + 3 of 4 consecutive keys; slot c ^ (((key >> 1) & 1) << 2) moves
//   keys 2 and 3 of each 4 to the other half of their rows.
__device__ __forceinline__ int k_slot(int key, int chunk) { return chunk ^ ((key >> 1) & 7); }
__device__ __forceinline__ int v_slot(int key, int chunk) { return chunk ^ (((key >> 1) & 1) << 2); }

typedef __attribute__((address_space(3))) void* LdsPtr;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
constexpr int kRows = kPrefillRowsPerWave;   // query rows per unit (two MFMA column blocks)

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* q_start;
  void* out;
  int64_t q_s0, q_s1;
  int64_t kv_s0, kv_s1, kv_s2;
  int64_t o_s0, o_s1;
  int64_t bt_stride;
  int32_t bt_contig;             // 1: NULL table, contiguous layout
  int32_t hkv, hq, group, max_blocks;
  float scale_log2;
};

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

template <int DT>
__device__ __forceinline__ f32x16_t mfma(const uint4& a, const uint4& b, const f32x16_t& c) {
  if constexpr (DT == NP_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Two fp32 values rounded to the input type and packed (low = first).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2_t x = {a, b};
  if constexpr (DT == NP_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2_t));
}

// l + the sum of the eight packed values of `x` (two per word), in fp32.
template <int DT>
__device__ __forceinline__ float sum_pairs(const uint4& x, float l) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (DT == NP_BF16)
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[k]),
                                          __builtin_bit_cast(bf16x2_t, 0x3f803f80u), l, false);
    else
      l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w[k]),
                                 __builtin_bit_cast(f16x2_t, 0x3c003c00u), l, false);
  }
  return l;
}

// Scores are finite or -inf here (masked slots are set to -inf by index
// before any max), so this file is built without NaN semantics and the max
// needs no canonicalisation: max(max(a, b), c) becomes one v_max3_f32. The
// running value goes first, so that a chain max3(m, x, y), max3(m', x', y')
// takes one instruction per two values (with the running value innermost on
// the other side, each pair of new values becomes a v_max_f32 of its own).
__device__ __forceinline__ float max3(float a, float b, float c) {
  return fmaxf(fmaxf(a, b), c);
}

__device__ __forceinline__ uint4 ld16(const void* base, int64_t elem_off) {
  return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem_off);
}

// Rows of units u0 .. units - 1 (unit u: query head kvh * G + u % G, rows
// 64 (u / G) .. of the sequence's chunk) set to NaN, as raw bits (this file
// is built without NaN semantics), 16 bytes per store; the whole workgroup
// takes part.
template <int DT>
__device__ __forceinline__ void nan_units(const PrefillParams& p, int row0, int n_q, int kvh,
                                          int G, int u0, int units) {
  const uint32_t w = DT == NP_BF16 ? 0x7fc07fc0u : 0x7e007e00u;
  const uint4 nan8 = make_uint4(w, w, w, w);
  const int per_unit = kRows * (kD / 8);
  for (int i = threadIdx.x; i < (units - u0) * per_unit; i += blockDim.x) {
    const int u = u0 + i / per_unit;
    const int r = (u / G) * kRows + (i % per_unit) / (kD / 8);
    const int c = 8 * (i % (kD / 8));
    if (r < n_q)
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + int64_t(row0 + r) * p.o_s0 +
                                int64_t(kvh * G + u % G) * p.o_s1 + c) = nan8;
  }
}

template <int DT, int BS>
__global__ __launch_bounds__(kPrefillWaves * kWaveSize) void paged_prefill_kernel(
    const PrefillParams p) {
  static_assert(BS == 16, "a wave stages one 16-slot block per key tile");
  constexpr int NU = kPrefillUnits;       // units (and waves per group)
  constexpr int NG = kPrefillWaves / NU;  // wave groups, taking alternate key tiles
  static_assert(NG == 2 && NU * BS == kKT, "two groups; one block per wave per tile");
  constexpr int QB = kRows / 32;          // 32-query column blocks per wave
  static_assert(QB == 2, "the step below pairs two query blocks");
  // kStages buffers per group of K and V tiles (tile 2j + g is group g's in
  // step j, in buffer j % kStages).
  constexpr int kTile = kKT * kD;
  // One LDS variable for all staged tiles (K stages, then V stages) and the
  // copy of the first kTabCache raw entries of the sequence's table row. (With
  // separate variables the compiler tags each access with its variable alone,
  // and would no longer see that a step's loads and reads use different
  // buffers of the same array.)
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStages * NG * kTile + 2 * kTabCache];
  auto& k_lds = *reinterpret_cast<uint16_t(*)[kStages][NG][kTile]>(lds);
  auto& v_lds = *reinterpret_cast<uint16_t(*)[kStages][NG][kTile]>(lds + kStages * NG * kTile);
  int32_t* const tab = reinterpret_cast<int32_t*>(lds + 2 * kStages * NG * kTile);

  const int kvh = blockIdx.x % p.hkv;
  // Tiles are launched largest first: later query rows see more keys under the
  // causal mask, so the longest workgroups start first and the shortest fill
  // the end of the launch (x runs over tiles in descending order).
  const int tile = int(gridDim.x) / p.hkv - 1 - int(blockIdx.x) / p.hkv;
  const int s = blockIdx.y;
  const int G = p.group;
  const int row0 = p.q_start[s];
  const int n_q = p.q_start[s + 1] - row0;
  const int L = p.lens[s];
  const int past = L - n_q;
  const int nqb = (n_q + kRows - 1) / kRows;
  const int units = G * nqb;
  // Device rows or lengths that this plan's grid does not cover (a plan made
  // for other host q_start or lengths), or that are invalid, get NaN rows
  // from the first launched tile instead of being left unwritten.
  const int plan_tiles = int(gridDim.x) / p.hkv;
  const bool bad = past < 0 || L > p.max_blocks * BS;
  const int first_uncovered = bad ? 0 : plan_tiles * NU;
  if (tile == plan_tiles - 1 && units > first_uncovered)
    nan_units<DT>(p, row0, n_q, kvh, G, first_uncovered, units);
  if (bad || tile * NU >= units) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
  const int grp = wave / NU;           // key tiles grp, grp + 2, grp + 4, ...
  const int wu = wave % NU;            // unit within the workgroup
  const int lane = threadIdx.x % kWaveSize;
  const int half = lane / 32;          // which 8 of a 16-wide k-step this lane feeds
  const int col = lane % 32;           // this lane's query column within a block

  // This wave's unit (head, 64-row query block); idle units' waves still stage K/V.
  const int unit = tile * NU + wu;
  const bool active = unit < units;
  const int h = active ? unit % G : 0;
  const int q0 = active ? (unit / G) * kRows : 0;
  // Last key any row of this unit sees, and of the whole workgroup.
  const int q_last = (q0 + kRows < n_q ? q0 + kRows : n_q) - 1;
  const int unit_last_key = active ? past + q_last : -1;
  int wg_last_unit = tile * NU + NU - 1;
  wg_last_unit = wg_last_unit < units ? wg_last_unit : units - 1;
  const int wg_q_last_blk = wg_last_unit / G;
  const int wg_q_last = ((wg_q_last_blk + 1) * kRows < n_q ? (wg_q_last_blk + 1) * kRows : n_q) - 1;
  const int n_tiles = (past + wg_q_last) / kKT + 1;
  const int n_steps = (n_tiles + NG - 1) / NG;
  const int unit_tiles = active ? unit_last_key / kKT + 1 : 0;

  // This lane's two queries (one per column block), in the four 16-channel
  // k-chunks (B operand of S^T).
  int my_q[QB];
  bool q_ok[QB];
  uint4 qreg[QB][kD / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    my_q[qb] = q0 + 32 * qb + col;
    q_ok[qb] = active && my_q[qb] < n_q;
    const int64_t qoff = int64_t(row0 + (q_ok[qb] ? my_q[qb] : 0)) * p.q_s0 +
                         int64_t(kvh * G + h) * p.q_s1 + 8 * half;
#pragma unroll
    for (int c = 0; c < kD / 16; ++c)
      qreg[qb][c] = q_ok[qb] ? ld16(p.q, qoff + 16 * c) : make_uint4(0, 0, 0, 0);
  }

  // Staging: in step j, wave w loads block w % NU of its group's tile 2j + w / NU
  // (16 keys, rows 16 (w % NU) ..) of K and of V straight into the tile
  // buffers, 8 rows per instruction; lane l fetches the chunk its LDS slot
  // holds under the swizzle. Blocks past the history re-read the last real
  // block; their rows, and the slots past the history in the last block, are
  // zeroed in V after the loads land (keys there get weight 0, and 0 times an
  // unwritten slot must not turn into NaN). K rows there are masked by score
  // selects.
  const TableRow bt_row = table_row(p.bt, p.bt_stride, s, p.max_blocks, p.bt_contig);
  int nb = (L + BS - 1) / BS;
  nb = nb < p.max_blocks ? nb : p.max_blocks;
  // Logical block wave (grp, wu) stages in step j (past the history: the last one).
  auto block_of = [&](int j) __attribute__((always_inline)) {
    const int blk = (NG * j + grp) * NU + wu;
    return blk < nb ? blk : nb - 1;
  };
  auto stage_issue = [&](int phys, const uint16_t* ksrc, const uint16_t* vsrc, uint16_t* kdst,
                         uint16_t* vdst) __attribute__((always_inline)) {
    const int64_t base = int64_t(phys) * p.kv_s0 + int64_t(kvh) * p.kv_s2;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int slot_row = 8 * n + lane / 8;       // slot of the block, row 16 wu + slot_row
      const int key = BS * wu + slot_row;          // row of the tile
      const int64_t src = base + int64_t(slot_row) * p.kv_s1;
      const int off = (BS * wu + 8 * n) * kD;      // wave-uniform destination row
      __builtin_amdgcn_global_load_lds(
          ksrc + src + 8 * k_slot(key, lane % 8),
          (LdsPtr)(kdst + off), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          vsrc + src + 8 * v_slot(key, lane % 8),
          (LdsPtr)(vdst + off), 16, 0, 0);
    }
  };
  auto stage_fix = [&](int j, uint16_t* vl) __attribute__((always_inline)) {
    const int key0 = ((NG * j + grp) * NU + wu) * BS;   // first key of the (unclamped) block
    if (key0 + BS <= L) return;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int slot_row = 8 * n + lane / 8;
      if (key0 + slot_row >= L)
        *reinterpret_cast<uint4*>(&vl[(BS * wu + slot_row) * kD + 8 * (lane % 8)]) =
            make_uint4(0, 0, 0, 0);
    }
  };
  // Wait until at most four (the next stage's) or none of this wave's loads
  // are outstanding (only the staging loads are in flight in the loop).
  auto wait_loads = [&](bool pending4) __attribute__((always_inline)) {
    if (pending4)
      __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4): the next stage's loads may fly on
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  };

  const float c = p.scale_log2;   // > 0
  const float rc = 1.0f / c;
  float m[QB], l[QB];          // running reference max (scaled, log2 units); lane's half-sum
  // Kept beside m, updated only when m moves: the exponent offset of the
  // weights (-m, or 0 while m is -inf) and the raw score above which m moves,
  // (m + kLazy) / c, so that neither costs instructions per tile.
  float nm[QB], thr[QB];
  f32x16_t acc[QB][kD / 32];   // O^T column blocks
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    nm[qb] = 0.0f;
    thr[qb] = -INFINITY;
    l[qb] = 0.0f;
#pragma unroll
    for (int cb = 0; cb < kD / 32; ++cb) acc[qb][cb] = f32x16_t{};
  }

  // Mask (keys past the query's position or past the history) on raw scores
  // and take the online-softmax step up to the rescale. The running max m
  // (scaled, log2 units) is lazy: it moves only when a score exceeds it by
  // more than kLazy, decided for the whole wave by a ballot, so the
  // cross-lane exchange and the rescale of acc are rare. Weights stay below
  // 2^kLazy, well inside the input type's range.
  auto softmax_head = [&](int kt, int qb, f32x16_t (&st)[2]) __attribute__((always_inline)) {
    const int key_base = kt * kKT;
    const bool need_mask = key_base + kKT - 1 > past + q0 + 32 * qb || key_base + kKT > L;
    if (need_mask) {
      // Last visible key of this row: past + row, and never past the history
      // (rows past the chunk end only exist as padding).
      const int lim = min(past + my_q[qb], L - 1) - key_base - 4 * half;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          st[b][i] = 32 * b + 8 * (i / 4) + (i % 4) <= lim ? st[b][i] : -INFINITY;
    }
    // Two chains of 7 (one per 32-key half), then 2 more: 16 instructions.
    float ma = max3(st[0][0], st[0][1], st[0][2]);
    float mb = max3(st[1][0], st[1][1], st[1][2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) {
      ma = max3(ma, st[0][i], st[0][i + 1]);
      mb = max3(mb, st[1][i], st[1][i + 1]);
    }
    const float mxr = max3(ma, mb, max3(st[0][15], st[1][15], st[1][15]));
    if (__ballot(mxr > thr[qb])) {
      const float mx = fmaxf(mxr, __shfl_xor(mxr, 32)) * c;   // same for the lane pair
      const bool move = mx > m[qb] + kLazy;                   // first tile: m = -inf
      const float alpha = move ? __builtin_amdgcn_exp2f(m[qb] - mx) : 1.0f;
      m[qb] = move ? mx : m[qb];
      nm[qb] = move ? -mx : nm[qb];
      thr[qb] = move ? (mx + kLazy) * rc : thr[qb];
      l[qb] *= alpha;
#pragma unroll
      for (int cb = 0; cb < kD / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[qb][cb][i] *= alpha;
    }
  };
  // P^T in the input type, packed for the B operand: k-step ks uses the
  // registers 8(ks%2) .. 8(ks%2)+7 of half ks/2. The row sum adds the same
  // rounded weights the product uses (v_dot2 against (1, 1)).
  // A lane whose scores so far were all masked still has m = -inf (a wave
  // group may start on a tile that some of its rows cannot see): its offset
  // nm is 0, so its weights are 0, not exp2(-inf + inf).
  auto weights = [&](int qb, int ks, const f32x16_t (&st)[2], uint4 (&pb)[4]) __attribute__((always_inline)) {
    const float neg_m = nm[qb];
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      e[j] = __builtin_amdgcn_exp2f(fmaf(st[ks / 2][8 * (ks % 2) + j], c, neg_m));
    pb[ks] = make_uint4(pack2<DT>(e[0], e[1]), pack2<DT>(e[2], e[3]),
                        pack2<DT>(e[4], e[5]), pack2<DT>(e[6], e[7]));
    l[qb] = sum_pairs<DT>(pb[ks], l[qb]);
  };

  // One key tile of this wave. The source pairs matrix-core work with
  // independent VALU work (an MFMA runs for many cycles after it issues; the
  // instructions after it, of this wave or of the other wave on the SIMD,
  // issue meanwhile):
  //   S^T of block 0
  //   softmax weights of block 0  | S^T of block 1
  //   softmax weights of block 1  | P.V of block 0
  //   P.V of block 1
  // and leaves the instruction order to the compiler's scheduler (fixing it
  // with scheduling barriers, and pinning each weight chunk in place, was
  // 2-4% slower).
  // Register j of k-step ks of P^T holds key 16 ks + 8 (j / 4) + 4 half + j % 4
  // of the tile; V^T is read in that order.
  auto tile_step = [&](int kt, const uint16_t* kl, const uint16_t* vl) __attribute__((always_inline)) {
    uint4 ka[2][kD / 16];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int k = 0; k < kD / 16; ++k) {
        const int key = 32 * b + col;
        ka[b][k] = *reinterpret_cast<const uint4*>(&kl[key * kD + 8 * k_slot(key, 2 * k + half)]);
      }
    f32x16_t s0[2], s1[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s0[b] = f32x16_t{};
#pragma unroll
      for (int k = 0; k < kD / 16; ++k) s0[b] = mfma<DT>(ka[b][k], qreg[0][k], s0[b]);
    }
    softmax_head(kt, 0, s0);
    uint4 pb0[4], pb1[4];
    s1[0] = f32x16_t{};
    s1[1] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      s1[0] = mfma<DT>(ka[0][ks], qreg[1][ks], s1[0]);
      s1[1] = mfma<DT>(ka[1][ks], qreg[1][ks], s1[1]);
      weights(0, ks, s0, pb0);
    }
    // V^T operand (A of O^T = V^T P^T): lane l needs keys 16 ks + 4 half + 0..3
    // and + 8 .. + 11 of channel 32 cb + l % 32. A transposing read hands lane t
    // of a 16-lane group element t % 4 of the 4-element vector addressed by lane
    // t / 4 + 4 j, for j = 0..3: so lane i of the group addresses key base + i / 4,
    // channels 32 cb + 16 ((l / 16) % 2) + 4 (i % 4) .. + 3.
    uint4 va[kD / 32][4];
    const int tr_row = (lane % 16) / 4;
    const int tr_col = 16 * ((lane / 16) % 2) + 4 * (lane % 4);
#pragma unroll
    for (int cb = 0; cb < kD / 32; ++cb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int key = 16 * ks + 8 * e + 4 * half + tr_row;
          const int ch = 32 * cb + tr_col;
          const uint16_t* a = &vl[key * kD + 8 * v_slot(key, ch / 8) + ch % 8];
          const i16x4_t t = __builtin_bit_cast(
              i16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (__attribute__((address_space(3))) i16x4_t*)a));
          w[2 * e] = uint32_t(uint16_t(t[0])) | (uint32_t(uint16_t(t[1])) << 16);
          w[2 * e + 1] = uint32_t(uint16_t(t[2])) | (uint32_t(uint16_t(t[3])) << 16);
        }
        va[cb][ks] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    softmax_head(kt, 1, s1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int cb = 0; cb < kD / 32; ++cb) acc[0][cb] = mfma<DT>(va[cb][ks], pb0[ks], acc[0][cb]);
      weights(1, ks, s1, pb1);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int cb = 0; cb < kD / 32; ++cb) acc[1][cb] = mfma<DT>(va[cb][ks], pb1[ks], acc[1][cb]);
  };

  // Step j: group g takes tile 2j + g from buffer j % kStages; the loads of
  // step j + 2 are issued before it (into the buffer step j - 1 used, free
  // since the last barrier) and must land, with step j + 1's, before step
  // j + 2; each step waits only for step j + 1's loads. One barrier per step.
  //
  // The three buffers of a step are distinct, and are passed as restrict
  // pointers: the compiler then knows the direct loads of step j + 2 do not
  // write what step j reads, and does not wait for them before every LDS read
  // (it would otherwise, and the prefetch would be lost). The loop-carried
  // order -- step j + 2's loads land before step j + 2 reads them -- is kept
  // by the explicit counter waits and barriers, which are plain s_barrier
  // (a fence would also wait for the loads in flight) after an LDS-counter
  // wait for this wave's own LDS writes.
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto step = [&](int j, const uint16_t* __restrict__ gk, const uint16_t* __restrict__ gv,
                  uint16_t* __restrict__ dma_k, uint16_t* __restrict__ dma_v,
                  const uint16_t* __restrict__ rd_k, const uint16_t* __restrict__ rd_v,
                  uint16_t* __restrict__ fix_v, const int32_t* __restrict__ tb) {
    if (j + 2 < n_steps) {
      const int b = block_of(j + 2);
      const int phys =
          b < kTabCache ? bt_row.phys(__builtin_amdgcn_readfirstlane(tb[b]), b) : bt_row[b];
      stage_issue(phys, gk, gv, dma_k, dma_v);
    }
    const int kt = NG * j + grp;
    if (kt < unit_tiles) tile_step(kt, rd_k, rd_v);
    if (j + 1 < n_steps) {
      wait_loads(j + 2 < n_steps);
      stage_fix(j + 1, fix_v);
    }
  };
  const uint16_t* gk = static_cast<const uint16_t*>(p.k);
  const uint16_t* gv = static_cast<const uint16_t*>(p.v);
  // The table entries are copied to LDS in the prologue, their reads issued
  // with the first two stages' loads (the copy then waits for both, once per
  // workgroup); a step reads its entry from LDS instead of waiting for a
  // scalar load of it from global memory.
  const int n_tab = nb < kTabCache ? nb : kTabCache;
  constexpr int kTabPerThread = kTabCache / (kPrefillWaves * kWaveSize);
  static_assert(kTabPerThread * kPrefillWaves * kWaveSize == kTabCache, "table copy");
  auto prologue = [&](const uint16_t* __restrict__ gk, const uint16_t* __restrict__ gv,
                      uint16_t* __restrict__ k0, uint16_t* __restrict__ v0,
                      uint16_t* __restrict__ k1, uint16_t* __restrict__ v1,
                      int32_t* __restrict__ tb) {
    stage_issue(bt_row[block_of(0)], gk, gv, k0, v0);
    int32_t tab_v[kTabPerThread];
#pragma unroll
    for (int i = 0; i < kTabPerThread; ++i) {
      const int b = int(threadIdx.x) + i * kPrefillWaves * kWaveSize;
      tab_v[i] = bt_row.raw(b < n_tab ? b : n_tab - 1);   // no branch: the wait stays at the write
    }
    if (1 < n_steps) stage_issue(bt_row[block_of(1)], gk, gv, k1, v1);
#pragma unroll
    for (int i = 0; i < kTabPerThread; ++i) tb[int(threadIdx.x) + i * kPrefillWaves * kWaveSize] = tab_v[i];
  };
  prologue(gk, gv, k_lds[0][grp], v_lds[0][grp], k_lds[1][grp], v_lds[1][grp], tab);
  wait_loads(1 < n_steps);
  stage_fix(0, v_lds[0][grp]);
  barrier();
  // Unrolled by the buffer count, so each step's buffers are fixed offsets
  // and the operand addresses need no per-step arithmetic.
  static_assert(kStages == 3, "unrolled by three");
  for (int j = 0; j < n_steps; j += 3) {
    step(j, gk, gv, k_lds[2][grp], v_lds[2][grp], k_lds[0][grp], v_lds[0][grp], v_lds[1][grp], tab);
    barrier();
    if (j + 1 >= n_steps) break;
    step(j + 1, gk, gv, k_lds[0][grp], v_lds[0][grp], k_lds[1][grp], v_lds[1][grp], v_lds[2][grp], tab);
    barrier();
    if (j + 2 >= n_steps) break;
    step(j + 2, gk, gv, k_lds[1][grp], v_lds[1][grp], k_lds[2][grp], v_lds[2][grp], v_lds[0][grp], tab);
    barrier();
  }

  // Merge the two groups' states of each unit through LDS (the staging
  // buffers are free now), one query block at a time: group 1 writes, group 0
  // combines and stores.
  float* xa = reinterpret_cast<float*>(&k_lds[0][0][0]);      // [NU][kD/32][16][64]
  float* xm = reinterpret_cast<float*>(&v_lds[0][0][0]);      // [NU][2][64]
  static_assert(NU * (kD / 32) * 16 * kWaveSize * 4 <= sizeof(k_lds), "merge space");
  static_assert(NU * 2 * kWaveSize * 4 <= sizeof(v_lds), "merge space");
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (grp == 1) {
      xm[(wu * 2 + 0) * kWaveSize + lane] = m[qb];
      xm[(wu * 2 + 1) * kWaveSize + lane] = l[qb];
#pragma unroll
      for (int cb = 0; cb < kD / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          xa[((wu * (kD / 32) + cb) * 16 + i) * kWaveSize + lane] = acc[qb][cb][i];
    }
    __syncthreads();
    if (grp == 0 && q_ok[qb]) {
      const float m1 = xm[(wu * 2 + 0) * kWaveSize + lane];
      const float l1 = xm[(wu * 2 + 1) * kWaveSize + lane];
      // m is shared by a lane pair (both halves of a query) and so is m1.
      const float mm = fmaxf(m[qb], m1);
      const float a0 = __builtin_amdgcn_exp2f(m[qb] - mm);   // 0 for a group that saw nothing
      const float a1 = __builtin_amdgcn_exp2f(m1 - mm);
      const float lh = l[qb] * a0 + l1 * a1;
      const float l_tot = lh + __shfl_xor(lh, 32);
      const float r = 1.0f / l_tot;
      const int64_t obase = int64_t(row0 + my_q[qb]) * p.o_s0 + int64_t(kvh * G + h) * p.o_s1;
#pragma unroll
      for (int cb = 0; cb < kD / 32; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * g + e;
            const float x1 = xa[((wu * (kD / 32) + cb) * 16 + i) * kWaveSize + lane];
            o[e] = (acc[qb][cb][i] * a0 + x1 * a1) * r;
          }
          const int ch = 32 * cb + 8 * g + 4 * half;
          const uint2 v = make_uint2(pack2<DT>(o[0], o[1]), pack2<DT>(o[2], o[3]));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + obase + ch) = v;
        }
    }
    __syncthreads();
  }
}

}  // namespace

}  // namespace np

using namespace np;

extern "C" np_status np_paged_attention_prefill(const np_paged_desc* desc,
                                                const np_plan_t* plan, const void* q,
                                                const void* k_pool, const void* v_pool,
                                                const int32_t* block_table,
                                                const int32_t* context_lens,
                                                const int32_t* q_start, void* out,
                                                void* workspace, size_t workspace_bytes,
                                                void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  np_status st = check_desc(desc);
  if (st != NP_OK) return st;
  st = check_pointers(desc, q, k_pool, v_pool, block_table, context_lens, out);
  if (st != NP_OK) return st;
  if (q_start == nullptr) return NP_ERR_NULL_PTR;
  if (reinterpret_cast<uintptr_t>(q_start) % 4 != 0) return NP_ERR_MISALIGNED;
  st = check_plan(desc, plan, 1);
  if (st != NP_OK) return st;
  const np_plan_core& c = plan->core;
  if ((c.dtype != NP_BF16 && c.dtype != NP_F16) || c.head_dim != kD || c.block_size != 16 ||
      c.group > kMaxGroup)
    return NP_ERR_UNSUPPORTED;
  PrefillParams prm{};
  prm.q = q;
  prm.k = k_pool;
  prm.v = v_pool;
  // A NULL table (contiguous layout) reads a stand-in row: see np_table.h.
  prm.bt = block_table ? block_table : context_lens;
  prm.bt_contig = block_table == nullptr;
  prm.lens = context_lens;
  prm.q_start = q_start;
  prm.out = out;
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
  prm.group = c.group;
  prm.max_blocks = c.max_blocks;
  const float scale = desc->scale > 0.0f ? desc->scale : 1.0f / std::sqrt(float(c.head_dim));
  prm.scale_log2 = scale * kLog2e;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  dim3 grid(c.grid[0], c.grid[1], c.grid[2]);
  if (c.dtype == NP_BF16)
    paged_prefill_kernel<NP_BF16, 16><<<grid, dim3(c.wg_size), 0, hs>>>(prm);
  else
    paged_prefill_kernel<NP_F16, 16><<<grid, dim3(c.wg_size), 0, hs>>>(prm);
  return hipGetLastError() == hipSuccess ? NP_OK : NP_ERR_HIP;
}
