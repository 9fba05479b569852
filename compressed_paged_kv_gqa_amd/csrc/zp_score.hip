// Per-token importance scores of requests about to be compressed (gfx950).
//
// Zipage (arXiv 2603.08743): App. C.2 Alg. 1 (block attention logits of the
// observation window with a causal mask on the last block; softmax over the
// whole sequence per query head, max over the GQA group, mean over the
// window), App. C.3 Alg. 2 (decayed max-reduce with the global score cache
// F), App. C.4 eq. (3) (max pooling after the global score), App. C.5 eq. (4),
// Fig. 11 and Alg. 3 (key redundancy: cosine similarities, diagonal and each
// column's last entry above p zeroed, row sums over the sequence length),
// App. C.7 (lightning: similarities inside each block only), App. C.8
// (tempered softmax of the redundancy), Sec. 4.2 (+inf on the window).
//
// Launches per call, parallel over (block, kv-head, layer x request):
//  A  score_block: one workgroup per block. The block's keys are staged in
//     LDS (XOR-swizzled 16-byte chunks, 16 loads in flight per thread), two
//     workgroups per CU. MFMA forms the window logits (g*w x b, per-row
//     partial max and sum of exp2) and, for the lightning redundancy, the
//     block's cosine matrix, whose epilogue only tracks each column's
//     highest row above p. The row sums themselves need no matrix: the sum
//     of row i of the cosine matrix is khat_i . (sum_j khat_j), minus the
//     diagonal and the zeroed entries.
//  F  (flash redundancy only) score_flash: one workgroup per column block;
//     the cosine blocks against every row block give each column its highest
//     row above p over the whole sequence (the row that Alg. 3's zero-out
//     tags single out, independent of the visiting order).
//  B  score_s0: per block again, merges the row statistics into log-sum-exp,
//     recomputes the logits, forms S0 (group max, window mean) and applies
//     the global score (reads F, writes the updated history to f_new).
//  C  finalize: per (request, kv-head): pooling, redundancy softmax over the
//     sequence, S - lambda R, +inf window -> scores.
// The window QK^T and the cosine matrices are dense contractions (bf16
// inputs, fp32 accumulation on MFMA 16x16x32; fp32 inputs use 16x16x4 f32).
#include <cmath>

#include "zp_device.h"
#include "zp_internal.h"

namespace zp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Row-major [rows][D] tile of T in LDS, stored as 16-byte chunks; chunk c of
// row r sits at position c ^ (r % SW) so that 16 lanes reading the same
// logical chunk of 16 consecutive rows hit distinct banks.
template <typename T, int D>
struct LdsTile {
  static constexpr int CH = D * (int)sizeof(T) / 16;  // chunks per row
  static constexpr int SW = CH < 16 ? CH : 16;
  static constexpr int ROWB = CH * 16;                // bytes per row
  static constexpr int EPC = 16 / (int)sizeof(T);     // elements per chunk
  __device__ static int chunk_pos(int r, int c) { return r * CH + (c ^ (r % SW)); }
};

// MFMA operand access. In both variants lane l works on row (l % 16) of the
// 16-row A tile / B tile and on the k-slice selected by l / 16; A and B use
// the same slice so the products pair equal head dimensions.
template <typename T, int D>
struct Mma;

template <int D>
struct Mma<bf16_t, D> {
  static constexpr int NKS = D / 32;  // k-steps of 32
  using op_t = bf16x8_t;
  __device__ static op_t lds(const char* base, int row, int ks, int lane) {
    using L = LdsTile<bf16_t, D>;
    const int c = ks * 4 + (lane >> 4);
    return __builtin_bit_cast(op_t, *reinterpret_cast<const uint4*>(base + L::chunk_pos(row, c) * 16));
  }
  __device__ static op_t glb(const bf16_t* rowp, int ks, int lane) {
    return __builtin_bit_cast(op_t, ld16(rowp + ks * 32 + (lane >> 4) * 8));
  }
  __device__ static floatx4 mma(op_t a, op_t b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <int D>
struct Mma<float, D> {
  static constexpr int NKS = D / 4;  // k-steps of 4
  using op_t = float;
  __device__ static op_t lds(const char* base, int row, int ks, int lane) {
    using L = LdsTile<float, D>;
    const int e = ks * 4 + (lane >> 4);
    return *reinterpret_cast<const float*>(base + L::chunk_pos(row, e >> 2) * 16 + (e & 3) * 4);
  }
  __device__ static op_t glb(const float* rowp, int ks, int lane) { return rowp[ks * 4 + (lane >> 4)]; }
  __device__ static floatx4 mma(op_t a, op_t b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Column tiles (16 tokens each) per wavefront: a block of b <= 256 tokens has
// at most 16 tiles, dealt to the 4 wavefronts as ct = wv, wv + 4, ...
constexpr int kCTW = 4;

// Sums of the zeroed cosines are accumulated by atomics whose order varies
// from run to run. They are kept in 64-bit fixed point (2^-40 units), where
// addition is exact and commutative, so every run gives the same bits. A
// cosine lies in [-1, 1] and a row collects at most one entry per column, so
// a sum stays below n * 2^40 < 2^63 for any n < 2^23.
constexpr double kFixScale = 1099511627776.0;  // 2^40
__device__ __forceinline__ unsigned long long to_fix(float c) {
  return static_cast<unsigned long long>(__double2ll_rn(static_cast<double>(c) * kFixScale));
}
__device__ __forceinline__ float from_fix(unsigned long long v) {
  return static_cast<float>(static_cast<double>(static_cast<long long>(v)) * (1.0 / kFixScale));
}

// Copies `rows` rows of D elements (contiguous in global memory) to an LDS
// tile with up to 16 loads in flight per thread.
template <typename T, int D>
__device__ void stage_rows(char* dst, const T* src, int rows, int tid) {
  using L = LdsTile<T, D>;
  constexpr int BATCH = 16;
  const int total = rows * L::CH;
  const char* s = reinterpret_cast<const char*>(src);
  for (int i0 = 0; i0 < total; i0 += 256 * BATCH) {
    uint4 v[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int i = i0 + u * 256 + tid;
      if (i < total) v[u] = ld16(s + (int64_t)i * 16);
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int i = i0 + u * 256 + tid;
      if (i < total) *reinterpret_cast<uint4*>(dst + L::chunk_pos(i / L::CH, i % L::CH) * 16) = v[u];
    }
  }
}

struct ScoreParams {
  const void* kc;
  const void* qwin;
  float* gscore;
  const int32_t* tables;
  const int32_t* num_blocks;
  const int32_t* qslot;
  const uint8_t* first;
  const uint8_t* lse_ok;  // per request: window rows' log-sum-exp in qwin_lse (or NULL)
  const float* qwin_lse;  // [L][max_slots][h_kv][g][w] natural-log LSE of window rows
  float* scores;
  float* f_new;  // updated global score (S1) per token, same layout as scores
  float* stats;  // [items][h_kv][max_blocks][R][2]  (max, sum) in the exp2 domain
  float* rbuf;   // [items][h_kv][max_blocks * b]     redundancy row sums / n
  unsigned long long* rsub;  // [items][h_kv][max_blocks * b] flash: zeroed entries, fixed point
  float* s1buf;  // [items][h_kv][max_blocks * b]     S1
  float* inv;    // [items][h_kv][max_blocks * b]     inverse key norms
  float* nrm;    // [items][h_kv][max_blocks * b]     key norms
  float* ksum;   // [items][h_kv][max_blocks][D]      sum of the block's unit keys
  uint32_t* err;
  int64_t scores_stride;
  int64_t kv_layer_elems, qwin_layer_elems, f_layer_elems, qlse_layer_elems;
  int32_t layer_begin, nreq, table_stride, max_blocks, num_blocks_total;
  int32_t b, h_kv, w, max_slots;
  float qk_scale;  // log2(e) / sqrt(d)
  float alpha, lambda_, inv_tau, p;
  int32_t pool_kernel;
  uint32_t flags;
};

// Resolves the (request, layer, block) of a page-level workgroup; returns the
// block id or -1 when the workgroup has nothing to do.
__device__ __forceinline__ int resolve_page(const ScoreParams& P, int pidx, int z, int* N_out,
                                            int* slot_out) {
  const int r = z % P.nreq;
  const int N = P.num_blocks[r];
  if (N <= 0 || pidx >= N) return -1;
  if (N > P.max_blocks || N > P.table_stride) {
    if (pidx == 0 && threadIdx.x == 0) flag_error(P.err, ZP_DEVERR_SEQ_LEN);
    return -1;
  }
  const int page = P.tables[(int64_t)r * P.table_stride + pidx];
  if (page < 0 || page >= P.num_blocks_total) {
    if (threadIdx.x == 0) flag_error(P.err, ZP_DEVERR_BLOCK_ID);
    return -1;
  }
  const int slot = P.qslot[r];
  if (slot < 0 || slot >= P.max_slots) {
    if (threadIdx.x == 0) flag_error(P.err, ZP_DEVERR_SLOT);
    return -1;
  }
  *N_out = N;
  *slot_out = slot;
  return page;
}

// The wavefront index as a scalar (wave-uniform) value, so that conditions on
// it compile to scalar branches rather than lane masks.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// B operands (keys as columns of the product) of this wavefront's column
// tiles ct = wv + 4 * cw, from an LDS tile or from global memory. Tiles past
// the block (b < 256) are clamped to the last one: they are computed but
// their results are discarded, which keeps the tile loops free of branches so
// that the MFMA chains of the four tiles interleave.
template <typename T, int D>
struct ColOps {
  using M = Mma<T, D>;
  typename M::op_t op[kCTW][M::NKS];
  __device__ static int tile(int wv, int cw, int CT) { return min(wv + 4 * cw, CT - 1); }
  __device__ void from_lds(const char* Ks, int CT, int wv, int lane) {
#pragma unroll
    for (int cw = 0; cw < kCTW; ++cw) {
      const int ct = tile(wv, cw, CT);
#pragma unroll
      for (int ks = 0; ks < M::NKS; ++ks) op[cw][ks] = M::lds(Ks, ct * 16 + (lane & 15), ks, lane);
    }
  }
  __device__ void from_global(const T* kblk, int CT, int wv, int lane) {
#pragma unroll
    for (int cw = 0; cw < kCTW; ++cw) {
      const int ct = tile(wv, cw, CT);
#pragma unroll
      for (int ks = 0; ks < M::NKS; ++ks)
        op[cw][ks] = M::glb(kblk + (int64_t)(ct * 16 + (lane & 15)) * D, ks, lane);
    }
  }
};

// acc[cw] = A (one 16-row tile, k-slices a[]) times the column tiles of B,
// with the k-steps of the four independent products interleaved.
template <typename T, int D>
__device__ __forceinline__ void mma_tiles(const typename Mma<T, D>::op_t* a, const ColOps<T, D>& B,
                                          floatx4* acc) {
  using M = Mma<T, D>;
#pragma unroll
  for (int cw = 0; cw < kCTW; ++cw) acc[cw] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < M::NKS; ++ks)
#pragma unroll
    for (int cw = 0; cw < kCTW; ++cw) acc[cw] = M::mma(a[ks], B.op[cw][ks], acc[cw]);
}

// Cosine tiles of row tile rt (keys of the LDS block Ks) against this
// wavefront's column tiles: for each column, remembers the highest row whose
// cosine exceeds p (global row index row_base + row). cos(k_i, k_j) > p is
// tested as k_i . k_j > p |k_i| |k_j| (zero-norm keys never pass, p >= 0);
// pnc[cw] = p |k_j| of the lane's column (+inf for tiles past the block).
// Rows grow with rt and with the register index, so the last hit is the
// highest. The diagonal of the block against itself is excluded when `self`.
// Branch-free, so that consecutive row tiles overlap in the schedule.
template <typename T, int D>
__device__ __forceinline__ void cosine_tile_rows(const char* Ks, const float* nrm_r, int rt,
                                                 const ColOps<T, D>& B, const float* pnc,
                                                 int wv, int lane, bool self, int row_base,
                                                 int* brow) {
  using M = Mma<T, D>;
  const int q = lane >> 4, cl = lane & 15;
  typename M::op_t a[M::NKS];
#pragma unroll
  for (int ks = 0; ks < M::NKS; ++ks) a[ks] = M::lds(Ks, rt * 16 + cl, ks, lane);
  const float4 nr = *reinterpret_cast<const float4*>(nrm_r + rt * 16 + 4 * q);
  const float nrv[4] = {nr.x, nr.y, nr.z, nr.w};
  floatx4 acc[kCTW];
  mma_tiles<T, D>(a, B, acc);
  const int row0 = row_base + rt * 16 + 4 * q;
#pragma unroll
  for (int cw = 0; cw < kCTW; ++cw) {
    const bool dg = self && wv + 4 * cw == rt;  // the block's diagonal tile
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float thr = dg && 4 * q + v == cl ? INFINITY : nrv[v] * pnc[cw];
      brow[cw] = acc[cw][v] > thr ? row0 + v : brow[cw];
    }
  }
}

// Highest row of each column over the four 4-row lane groups; valid in all
// lanes (column ct * 16 + lane % 16).
__device__ __forceinline__ void best_over_groups(int* brow) {
#pragma unroll
  for (int cw = 0; cw < kCTW; ++cw) {
    brow[cw] = max(brow[cw], shfl_xor_i(brow[cw], 16));
    brow[cw] = max(brow[cw], shfl_xor_i(brow[cw], 32));
  }
}

// Dot product of two rows of D elements (fp32 accumulation).
template <typename T, int D>
__device__ __forceinline__ float row_dot(const T* x, const T* y) {
  float d = 0.f;
  if constexpr (sizeof(T) == 2) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll 4
    for (int c = 0; c < D / 8; ++c) {
      const uint4 u = ld16(x + c * 8), v = ld16(y + c * 8);
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.x), __builtin_bit_cast(bf2, v.x), d, false);
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.y), __builtin_bit_cast(bf2, v.y), d, false);
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.z), __builtin_bit_cast(bf2, v.z), d, false);
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.w), __builtin_bit_cast(bf2, v.w), d, false);
    }
  } else {
#pragma unroll 4
    for (int e = 0; e < D; ++e) d = fmaf(x[e], y[e], d);
  }
  return d;
}

// Same for two rows of an LDS tile.
template <typename T, int D>
__device__ __forceinline__ float lds_row_dot(const char* Ks, int r1, int r2) {
  using L = LdsTile<T, D>;
  float d = 0.f;
#pragma unroll 4
  for (int c = 0; c < L::CH; ++c) {
    const uint4 u = *reinterpret_cast<const uint4*>(Ks + L::chunk_pos(r1, c) * 16);
    const uint4 v = *reinterpret_cast<const uint4*>(Ks + L::chunk_pos(r2, c) * 16);
    if constexpr (sizeof(T) == 2) {
      typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.x), __builtin_bit_cast(bf2, v.x), d, false);
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.y), __builtin_bit_cast(bf2, v.y), d, false);
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.z), __builtin_bit_cast(bf2, v.z), d, false);
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.w), __builtin_bit_cast(bf2, v.w), d, false);
    } else {
      d = fmaf(__uint_as_float(u.x), __uint_as_float(v.x), d);
      d = fmaf(__uint_as_float(u.y), __uint_as_float(v.y), d);
      d = fmaf(__uint_as_float(u.z), __uint_as_float(v.z), d);
      d = fmaf(__uint_as_float(u.w), __uint_as_float(v.w), d);
    }
  }
  return d;
}

// Dot product of row r of an LDS tile with an fp32 vector v[D].
template <typename T, int D>
__device__ __forceinline__ float lds_row_dot_f32(const char* Ks, int r, const float* v) {
  using L = LdsTile<T, D>;
  float d = 0.f;
#pragma unroll 4
  for (int c = 0; c < L::CH; ++c) {
    const uint4 x = *reinterpret_cast<const uint4*>(Ks + L::chunk_pos(r, c) * 16);
    float f[L::EPC];
    Vec16<T>::unpack(x, f);
#pragma unroll
    for (int e = 0; e < L::EPC; ++e) d = fmaf(f[e], v[c * L::EPC + e], d);
  }
  return d;
}

// ---------------------------------------------------------------------------
// S0 of one block (App. C.2) and the global score (Alg. 2), given the
// log-sum-exp of every window row.
// ---------------------------------------------------------------------------
// For this wavefront's column tiles (B) and the window rows' log-sum-exp in
// the exp2 domain (lse2[R], LDS), forms P = exp2(logit - lse2) with the causal
// mask of the last block, S0 = window mean of the group max, applies the
// global score and writes f_new and S1. qop(rt, a) fills the A operands of row
// tile rt. W16: the window is 16 slots, so row tile rt holds query head rt and
// its 16 rows are the window positions: the group max is a max over row tiles
// in registers and the window mean a sum over the lane's rows and lane
// groups. Otherwise the probabilities of a column tile go through LDS (ptile,
// [4][R][16] floats).
template <typename T, int D, int R, bool W16, typename QOp>
__device__ __forceinline__ void s0_columns(const ScoreParams& P, const ColOps<T, D>& B, QOp qop,
                                           const float* lse2, float* ptile, int wv, int lane,
                                           int CT, bool last, bool first, int layer, int page,
                                           int pidx, int64_t zh, int h) {
  using M = Mma<T, D>;
  constexpr int RT = R / 16;
  const int q = lane >> 4, cl = lane & 15;
  const int b = P.b;
  auto emit = [&](int col, float s0) {
    float s1 = s0;
    if (P.flags & ZP_SCORE_GLOBAL) {
      // F is read only: blocks may be shared by several requests.
      if (!first && !last) {
        const float f = P.alpha * P.gscore[layer * P.f_layer_elems + ((int64_t)page * P.h_kv + h) * b + col];
        s1 = (P.flags & ZP_SCORE_GLOBAL_SUM) ? f + s0 : fmaxf(f, s0);
      }
      P.f_new[zh * P.scores_stride + (int64_t)pidx * b + col] = s1;
    }
    P.s1buf[zh * ((int64_t)P.max_blocks * b) + (int64_t)pidx * b + col] = s1;
  };
  const float sc2 = P.qk_scale;

  if constexpr (W16) {
    float pm[kCTW][4];
#pragma unroll
    for (int cw = 0; cw < kCTW; ++cw)
#pragma unroll
      for (int v = 0; v < 4; ++v) pm[cw][v] = 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      typename M::op_t a[M::NKS];
      qop(rt, a);
      floatx4 acc[kCTW];
      mma_tiles<T, D>(a, B, acc);
      const float4 l4 = *reinterpret_cast<const float4*>(lse2 + rt * 16 + 4 * q);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
      for (int cw = 0; cw < kCTW; ++cw)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          pm[cw][v] = fmaxf(pm[cw][v], __builtin_amdgcn_exp2f(fmaf(acc[cw][v], sc2, -lv[v])));
    }
#pragma unroll
    for (int cw = 0; cw < kCTW; ++cw) {
      const int ct = wv + 4 * cw;
      if (ct >= CT) continue;  // scalar
      if (last) {              // scalar: causal mask, window slot u = 4q + v
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (ct * 16 + cl > b - 16 + 4 * q + v) pm[cw][v] = 0.f;
      }
      float s = (pm[cw][0] + pm[cw][1]) + (pm[cw][2] + pm[cw][3]);
      s += shfl_xor_f(s, 16);
      s += shfl_xor_f(s, 32);
      if (q == 0) emit(ct * 16 + cl, s * (1.0f / 16.0f));
    }
  } else {
    const int G = R / P.w;
    float* ptw = ptile + wv * R * 16;
#pragma unroll
    for (int cw = 0; cw < kCTW; ++cw) {
      const int ct = wv + 4 * cw;
      if (ct >= CT) continue;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        typename M::op_t a[M::NKS];
        qop(rt, a);
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < M::NKS; ++ks) acc = M::mma(a[ks], B.op[cw][ks], acc);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = rt * 16 + 4 * q + v;
          const int col = ct * 16 + cl;
          const int u = row % P.w;
          float pv = exp2f(acc[v] * sc2 - lse2[row]);
          if (last && col > b - P.w + u) pv = 0.f;
          ptw[row * 16 + cl] = pv;
        }
      }
      // Within a wavefront LDS writes and reads are ordered; no barrier needed.
      if (lane < 16) {
        float s0 = 0.f;
        for (int u = 0; u < P.w; ++u) {
          float mx = 0.f;
          for (int gi = 0; gi < G; ++gi) mx = fmaxf(mx, ptw[(gi * P.w + u) * 16 + lane]);
          s0 += mx;
        }
        emit(ct * 16 + lane, s0 / (float)P.w);
      }
    }
  }
}

// Whether request r's window rows come with their log-sum-exp.
__device__ __forceinline__ bool lse_given(const ScoreParams& P, int r) {
  return P.lse_ok && P.qwin_lse && P.lse_ok[r] != 0;
}

// ---------------------------------------------------------------------------
// Phase A: row statistics of the window logits; key norms and unit-key sums;
// lightning redundancy rows.
// ---------------------------------------------------------------------------
template <typename T, int D, int R>
__global__ __launch_bounds__(256, 2) void score_block_kernel(ScoreParams P) {
  using L = LdsTile<T, D>;
  using M = Mma<T, D>;
  constexpr int RT = R / 16;
  extern __shared__ __align__(16) char smem[];
  const int b = P.b;
  char* Ks = smem;                                            // [b][D]
  float* inv_s = reinterpret_cast<float*>(Ks + b * L::ROWB);  // [b]
  float* nrm_s = inv_s + b;                                   // [b]
  float* ksum_s = nrm_s + b;                                  // [D]
  float* wstat = ksum_s + D;                                  // [4][R][2]
  // [b] fixed-point sums (8-byte aligned: every array above has an even
  // number of 4-byte entries and Ks is a multiple of 16 bytes)
  unsigned long long* sub = reinterpret_cast<unsigned long long*>(wstat + 4 * R * 2);
  int* istar = reinterpret_cast<int*>(sub + b);               // [b]
  float* lse2 = reinterpret_cast<float*>(istar + b);          // [R]
  float* ptile = lse2 + R;     // [4][R][16], window LSE given and window != 16 only

  const int pidx = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
  int N, slot;
  const int page = resolve_page(P, pidx, z, &N, &slot);
  if (page < 0) return;
  const int layer = P.layer_begin + z / P.nreq;
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int q = lane >> 4, cl = lane & 15;
  const bool last = pidx == N - 1;
  const int n = N * b;
  const int CT = b / 16;
  const int64_t zh = (int64_t)z * P.h_kv + h;
  const bool redun = (P.flags & ZP_SCORE_REDUNDANCY) != 0;
  const bool flash = redun && (P.flags & ZP_SCORE_REDUNDANCY_FLASH);

  const T* kpage = reinterpret_cast<const T*>(P.kc) + layer * P.kv_layer_elems +
                   ((int64_t)page * P.h_kv + h) * b * D;
  const T* qrows = reinterpret_cast<const T*>(P.qwin) + layer * P.qwin_layer_elems +
                   ((int64_t)slot * P.h_kv + h) * R * D;
  stage_rows<T, D>(Ks, kpage, b, tid);
  if (tid < b) sub[tid] = 0ull;
  // Window-query operands (A) of every row tile, in flight while the key
  // norms are formed (fp32 operands take 4x the registers: those are loaded
  // per row tile).
  constexpr bool PREQ = sizeof(T) == 2;
  typename M::op_t qa[PREQ ? RT : 1][M::NKS];
  if constexpr (PREQ) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ks = 0; ks < M::NKS; ++ks)
        qa[rt][ks] = M::glb(qrows + (int64_t)(rt * 16 + cl) * D, ks, lane);
  }
  __syncthreads();

  // Key norms, and the sum of the block's unit keys (thread = chunk c of the
  // row, rows rg, rg + RG, ...; the RG partial sums of a chunk sit in
  // consecutive lanes).
  float mainr = 0.f;
  if (redun) {
    float ss = 0.f;
    if (tid < b) {
      ss = lds_row_dot<T, D>(Ks, tid, tid);
      inv_s[tid] = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
      nrm_s[tid] = sqrtf(ss);
    }
    __syncthreads();
    constexpr int RG = 256 / L::CH;
    const int c = tid / RG, rg = tid % RG;
    float acc[L::EPC];
#pragma unroll
    for (int e = 0; e < L::EPC; ++e) acc[e] = 0.f;
    for (int r = rg; r < b; r += RG) {
      const uint4 x = *reinterpret_cast<const uint4*>(Ks + L::chunk_pos(r, c) * 16);
      float f[L::EPC];
      Vec16<T>::unpack(x, f);
      const float iv = inv_s[r];
#pragma unroll
      for (int e = 0; e < L::EPC; ++e) acc[e] = fmaf(f[e], iv, acc[e]);
    }
#pragma unroll
    for (int e = 0; e < L::EPC; ++e) acc[e] = group_sum<RG>(acc[e]);
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < L::EPC; ++e) ksum_s[c * L::EPC + e] = acc[e];
    }
    __syncthreads();
    float* ks_out = P.ksum + (zh * P.max_blocks + pidx) * D;
    for (int e = tid; e < D; e += 256) ks_out[e] = ksum_s[e];
    if (tid < b) {
      P.inv[zh * ((int64_t)P.max_blocks * b) + (int64_t)pidx * b + tid] = inv_s[tid];
      P.nrm[zh * ((int64_t)P.max_blocks * b) + (int64_t)pidx * b + tid] = nrm_s[tid];
      // row sum of the block's cosine matrix without its diagonal
      if (!flash) {
        const float iv = inv_s[tid];
        mainr = iv * lds_row_dot_f32<T, D>(Ks, tid, ksum_s) - iv * iv * ss;
      }
    }
  }

  // Window logits: B operands = this wavefront's column tiles of the block.
  ColOps<T, D> B;
  B.from_lds(Ks, CT, wv, lane);
  const int r = z % P.nreq;
  if (lse_given(P, r)) {
    // The window rows' log-sum-exp came with the queries (the attention pass
    // that produced each window token saw exactly its causal row): S0 and the
    // global score straight from this block, no statistics pass.
    if (tid < R)
      lse2[tid] = P.qwin_lse[layer * P.qlse_layer_elems + ((int64_t)slot * P.h_kv + h) * R + tid] * kLog2e;
    __syncthreads();
    auto qop = [&](int rt, typename M::op_t* a) {
      if constexpr (PREQ) {
#pragma unroll
        for (int ks = 0; ks < M::NKS; ++ks) a[ks] = qa[rt][ks];
      } else {
#pragma unroll
        for (int ks = 0; ks < M::NKS; ++ks) a[ks] = M::glb(qrows + (int64_t)(rt * 16 + cl) * D, ks, lane);
      }
    };
    if (P.w == 16)
      s0_columns<T, D, R, true>(P, B, qop, lse2, ptile, wv, lane, CT, last, P.first[r] != 0,
                                layer, page, pidx, zh, h);
    else
      s0_columns<T, D, R, false>(P, B, qop, lse2, ptile, wv, lane, CT, last, P.first[r] != 0,
                                 layer, page, pidx, zh, h);
  } else {
  // Row statistics in the exp2 domain of the scaled logits: per row the max
  // (M * scale) and the sum of exp2((x - M) * scale) over the block.
  const float sc2 = P.qk_scale;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if constexpr (!PREQ) {
#pragma unroll
      for (int ks = 0; ks < M::NKS; ++ks)
        qa[0][ks] = M::glb(qrows + (int64_t)(rt * 16 + cl) * D, ks, lane);
    }
    floatx4 acc[kCTW];
    mma_tiles<T, D>(qa[PREQ ? rt : 0], B, acc);
#pragma unroll
    for (int cw = 0; cw < kCTW; ++cw) {
      const int ct = wv + 4 * cw;
      if (ct >= CT) {  // scalar
        acc[cw] = floatx4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      } else if (last) {  // scalar: causal mask of the window rows in the last block
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int u = (rt * 16 + 4 * q + v) % P.w;
          if (ct * 16 + cl > b - P.w + u) acc[cw][v] = -INFINITY;
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = rt * 16 + 4 * q + v;
      float mx = acc[0][v];
#pragma unroll
      for (int cw = 1; cw < kCTW; ++cw) mx = fmaxf(mx, acc[cw][v]);
      const float Mx = group_max<16>(mx);
      const float ms = Mx == -INFINITY ? 0.f : Mx * sc2;
      float s = 0.f;
#pragma unroll
      for (int cw = 0; cw < kCTW; ++cw) s += __builtin_amdgcn_exp2f(fmaf(acc[cw][v], sc2, -ms));
      s = group_sum<16>(s);
      if (cl == 0) {
        wstat[(wv * R + row) * 2] = Mx == -INFINITY ? -INFINITY : ms;
        wstat[(wv * R + row) * 2 + 1] = s;
      }
    }
  }
  __syncthreads();
  if (tid < R) {
    float Mx = -INFINITY;
    for (int w2 = 0; w2 < 4; ++w2) Mx = fmaxf(Mx, wstat[(w2 * R + tid) * 2]);
    float S = 0.f;
    if (Mx != -INFINITY)
      for (int w2 = 0; w2 < 4; ++w2)
        S += wstat[(w2 * R + tid) * 2 + 1] * exp2f(wstat[(w2 * R + tid) * 2] - Mx);
    float* st = P.stats + ((zh * P.max_blocks + pidx) * R + tid) * 2;
    st[0] = Mx;
    st[1] = S;
  }
  }

  if (!redun) return;
  float* rrow = P.rbuf + zh * ((int64_t)P.max_blocks * b) + (int64_t)pidx * b;
  if (flash) {
    // score_flash_kernel accumulates the zeroed entries into these rows next.
    if (tid < b) P.rsub[zh * ((int64_t)P.max_blocks * b) + (int64_t)pidx * b + tid] = 0ull;
    return;
  }
  // Lightning redundancy: cosines inside this block only.
  int brow[kCTW];
  float pnc[kCTW];
#pragma unroll
  for (int cw = 0; cw < kCTW; ++cw) {
    brow[cw] = -1;
    pnc[cw] = wv + 4 * cw < CT ? P.p * nrm_s[(wv + 4 * cw) * 16 + cl] : INFINITY;
  }
  for (int rt = 0; rt < CT; ++rt)
    cosine_tile_rows<T, D>(Ks, nrm_s, rt, B, pnc, wv, lane, true, 0, brow);
  best_over_groups(brow);
  if (q == 0) {
#pragma unroll
    for (int cw = 0; cw < kCTW; ++cw) {
      const int ct = wv + 4 * cw;
      if (ct < CT) istar[ct * 16 + cl] = brow[cw];
    }
  }
  __syncthreads();
  // The zeroed entry of column j is cos(k_i*, k_j), subtracted from row i*.
  if (tid < b) {
    const int is = istar[tid];
    if (is >= 0) atomicAdd(&sub[is], to_fix(lds_row_dot<T, D>(Ks, is, tid) * inv_s[is] * inv_s[tid]));
  }
  __syncthreads();
  if (tid < b) rrow[tid] = (mainr - from_fix(sub[tid])) / (float)n;
}

// ---------------------------------------------------------------------------
// Flash redundancy (Zipage Alg. 3): one workgroup per column block m. Every
// row block i is staged in turn and its cosines against the columns of m are
// formed; each column keeps its highest row above p over the whole sequence
// (the entry Alg. 3 zeroes when it scans the row blocks from the last one
// with a zero-out tag per column). Row i's sum over the whole sequence is
// khat_i . (sum of all unit keys) minus its diagonal; the zeroed entries are
// subtracted from the rows they sit in.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256, 2) void score_flash_kernel(ScoreParams P) {
  using L = LdsTile<T, D>;
  extern __shared__ __align__(16) char smem[];
  const int b = P.b;
  char* Ks = smem;                                            // [b][D]
  float* stot = reinterpret_cast<float*>(Ks + b * L::ROWB);   // [D]

  const int m = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
  int N, slot;
  const int page_m = resolve_page(P, m, z, &N, &slot);
  if (page_m < 0) return;
  const int r = z % P.nreq;
  const int layer = P.layer_begin + z / P.nreq;
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int q = lane >> 4, cl = lane & 15;
  const int CT = b / 16;
  const int64_t zh = (int64_t)z * P.h_kv + h;
  const int32_t* tab = P.tables + (int64_t)r * P.table_stride;
  for (int i = 0; i < N; ++i) {          // all block ids were checked by phase A
    const int pg = tab[i];
    if (pg < 0 || pg >= P.num_blocks_total) return;
  }
  const T* kbase = reinterpret_cast<const T*>(P.kc) + layer * P.kv_layer_elems;
  const float* invz = P.inv + zh * ((int64_t)P.max_blocks * b);
  const float* nrmz = P.nrm + zh * ((int64_t)P.max_blocks * b);
  const float* ksz = P.ksum + zh * P.max_blocks * D;
  for (int e = tid; e < D; e += 256) {
    float s = 0.f;
    for (int i = 0; i < N; ++i) s += ksz[(int64_t)i * D + e];
    stot[e] = s;
  }
  const T* kpm = kbase + ((int64_t)page_m * P.h_kv + h) * b * D;
  ColOps<T, D> B;
  B.from_global(kpm, CT, wv, lane);
  int brow[kCTW];
  float pnc[kCTW];
#pragma unroll
  for (int cw = 0; cw < kCTW; ++cw) {
    brow[cw] = -1;
    pnc[cw] = wv + 4 * cw < CT ? P.p * nrmz[(int64_t)m * b + (wv + 4 * cw) * 16 + cl] : INFINITY;
  }
  float mainr = 0.f;
  for (int i = 0; i < N; ++i) {          // ascending rows: the last hit is the highest
    __syncthreads();                     // the previous block is no longer read
    stage_rows<T, D>(Ks, kbase + ((int64_t)tab[i] * P.h_kv + h) * b * D, b, tid);
    __syncthreads();
    if (i == m && tid < b) {
      const float iv = invz[(int64_t)m * b + tid];
      mainr = iv * lds_row_dot_f32<T, D>(Ks, tid, stot) - iv * iv * lds_row_dot<T, D>(Ks, tid, tid);
    }
    const float* nrm_r = nrmz + (int64_t)i * b;
    for (int rt = 0; rt < CT; ++rt)
      cosine_tile_rows<T, D>(Ks, nrm_r, rt, B, pnc, wv, lane, i == m, i * b, brow);
  }
  best_over_groups(brow);
  unsigned long long* rs = P.rsub + zh * ((int64_t)P.max_blocks * b);
  if (q == 0) {
#pragma unroll
    for (int cw = 0; cw < kCTW; ++cw) {
      const int ct = wv + 4 * cw;
      const int is = brow[cw];
      if (ct < CT && is >= 0) {
        const int j = ct * 16 + cl;
        const T* ki = kbase + ((int64_t)tab[is / b] * P.h_kv + h) * b * D + (int64_t)(is % b) * D;
        const float c = row_dot<T, D>(ki, kpm + (int64_t)j * D) * invz[is] * invz[(int64_t)m * b + j];
        atomicAdd(rs + is, to_fix(c));
      }
    }
  }
  // Rows of block m belong to this workgroup alone; finalize subtracts the
  // zeroed entries (rsub) once every column block has added its own.
  if (tid < b) P.rbuf[zh * ((int64_t)P.max_blocks * b) + (int64_t)m * b + tid] = mainr;
}

// ---------------------------------------------------------------------------
// Phase B (requests without window log-sum-exp): merges the per-block row
// statistics into log-sum-exp, recomputes the logits, S0 and global score.
// ---------------------------------------------------------------------------
template <typename T, int D, int R, bool W16>
__global__ __launch_bounds__(256, 2) void score_s0_kernel(ScoreParams P) {
  using L = LdsTile<T, D>;
  using M = Mma<T, D>;
  extern __shared__ __align__(16) char smem[];
  char* Qs = smem;                                           // [R][D]
  float* lse2 = reinterpret_cast<float*>(Qs + R * L::ROWB);  // [R]
  float* ptile = lse2 + R;                        // [4][R][16] (general window only)

  const int pidx = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
  int N, slot;
  const int page = resolve_page(P, pidx, z, &N, &slot);
  if (page < 0) return;
  const int r = z % P.nreq;
  if (lse_given(P, r)) return;  // done by phase A
  const int layer = P.layer_begin + z / P.nreq;
  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int cl = lane & 15;
  const int b = P.b;
  const int CT = b / 16;
  const bool last = pidx == N - 1;
  const int64_t zh = (int64_t)z * P.h_kv + h;

  const T* kpage = reinterpret_cast<const T*>(P.kc) + layer * P.kv_layer_elems +
                   ((int64_t)page * P.h_kv + h) * b * D;
  const T* qrows = reinterpret_cast<const T*>(P.qwin) + layer * P.qwin_layer_elems +
                   ((int64_t)slot * P.h_kv + h) * R * D;
  ColOps<T, D> B;
  B.from_global(kpage, CT, wv, lane);
  stage_rows<T, D>(Qs, qrows, R, tid);
  if (tid < R) {
    const float* st = P.stats + (zh * P.max_blocks) * R * 2 + tid * 2;
    float Mx = -INFINITY;
    for (int i = 0; i < N; ++i) Mx = fmaxf(Mx, st[(int64_t)i * R * 2]);
    float S = 0.f;
    for (int i = 0; i < N; ++i) S += st[(int64_t)i * R * 2 + 1] * exp2f(st[(int64_t)i * R * 2] - Mx);
    lse2[tid] = Mx + log2f(S);
  }
  __syncthreads();
  auto qop = [&](int rt, typename M::op_t* a) {
#pragma unroll
    for (int ks = 0; ks < M::NKS; ++ks) a[ks] = M::lds(Qs, rt * 16 + cl, ks, lane);
  };
  s0_columns<T, D, R, W16>(P, B, qop, lse2, ptile, wv, lane, CT, last, P.first[r] != 0, layer,
                           page, pidx, zh, h);
}

// ---------------------------------------------------------------------------
// Phase C: pooling, redundancy softmax, combination, window.
// ---------------------------------------------------------------------------
__device__ float block_reduce(float v, bool is_max, float* red) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  v = is_max ? group_max<64>(v) : group_sum<64>(v);
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  float t = red[0];
  for (int i = 1; i < 4; ++i) t = is_max ? fmaxf(t, red[i]) : t + red[i];
  return t;
}

__global__ __launch_bounds__(256) void score_finalize_kernel(ScoreParams P) {
  __shared__ float red[4];
  const int h = blockIdx.x, z = blockIdx.y;
  const int r = z % P.nreq;
  const int N = P.num_blocks[r];
  if (N <= 0 || N > P.max_blocks || N > P.table_stride) return;
  const int slot = P.qslot[r];
  if (slot < 0 || slot >= P.max_slots) return;
  for (int i = 0; i < N; ++i) {
    const int pg = P.tables[(int64_t)r * P.table_stride + i];
    if (pg < 0 || pg >= P.num_blocks_total) return;  // phases A/B flagged it
  }
  const int tid = threadIdx.x;
  const int n = N * P.b;
  const int64_t zh = (int64_t)z * P.h_kv + h;
  const float* s1 = P.s1buf + zh * ((int64_t)P.max_blocks * P.b);
  float* rr = P.rbuf + zh * ((int64_t)P.max_blocks * P.b);
  float* out = P.scores + zh * P.scores_stride;
  const bool first = P.first[r] != 0;
  const bool pool = (P.flags & ZP_SCORE_POOL) && (first || !(P.flags & ZP_SCORE_POOL_FIRST_ONLY));
  const bool redun = (P.flags & ZP_SCORE_REDUNDANCY) != 0;
  const int half = P.pool_kernel / 2;
  const float c2 = P.inv_tau * kLog2e;  // softmax(r / tau) in the exp2 domain

  float mx = -INFINITY, sum = 0.f;
  if (redun && (P.flags & ZP_SCORE_REDUNDANCY_FLASH)) {
    // flash: row sum over the whole sequence minus its zeroed entries, / n
    // (each thread keeps the same tokens t in every pass below)
    const unsigned long long* rs = P.rsub + zh * ((int64_t)P.max_blocks * P.b);
    for (int t = tid; t < n; t += 256) rr[t] = (rr[t] - from_fix(rs[t])) / (float)n;
  }
  if (redun) {
    float m = -INFINITY;
    for (int t = tid; t < n; t += 256) m = fmaxf(m, rr[t] * c2);
    mx = block_reduce(m, true, red);
    float s = 0.f;
    for (int t = tid; t < n; t += 256) s += exp2f(rr[t] * c2 - mx);
    sum = block_reduce(s, false, red);
  }
  const float inv_sum = redun ? 1.0f / sum : 0.f;
  for (int t = tid; t < n; t += 256) {
    float s = s1[t];
    if (pool) {
      const int lo = max(0, t - half), hi = min(n - 1, t + half);
      for (int i = lo; i <= hi; ++i) s = fmaxf(s, s1[i]);
    }
    if (redun) s -= P.lambda_ * (exp2f(rr[t] * c2 - mx) * inv_sum);
    if (t >= n - P.w) s = INFINITY;
    out[t] = s;
  }
}

constexpr size_t kMaxLds = 160 * 1024;  // gfx950 LDS per workgroup

template <typename T, int D, int R>
static zp_status launch_score(const ScoreParams& P, int items, hipStream_t s) {
  using L = LdsTile<T, D>;
  const int b = P.b;
  const bool w16 = P.w == 16;
  const size_t ptileA = (P.lse_ok && !w16) ? size_t(4) * R * 16 : 0;
  const size_t smemA = size_t(b) * L::ROWB +
                       sizeof(float) * (2 * b + D + 4 * R * 2 + 3 * b + R + ptileA);
  const size_t smemF = size_t(b) * L::ROWB + sizeof(float) * D;
  const size_t smemB = size_t(R) * L::ROWB + sizeof(float) * (R + (w16 ? 0 : 4 * R * 16));
  const bool flash = (P.flags & ZP_SCORE_REDUNDANCY) && (P.flags & ZP_SCORE_REDUNDANCY_FLASH);
  if (smemA > kMaxLds || smemB > kMaxLds || (flash && smemF > kMaxLds))
    return fail(ZP_EINVAL, "zp_score_tokens: block_size %d with this dtype/head_dim needs %zu "
                "bytes of LDS (max %zu)", b, smemA, kMaxLds);
  auto kA = score_block_kernel<T, D, R>;
  auto kF = score_flash_kernel<T, D>;
  auto kB = w16 ? score_s0_kernel<T, D, R, true> : score_s0_kernel<T, D, R, false>;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kA),
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(smemA)) != hipSuccess ||
      (flash && hipFuncSetAttribute(reinterpret_cast<const void*>(kF),
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    int(smemF)) != hipSuccess) ||
      hipFuncSetAttribute(reinterpret_cast<const void*>(kB),
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(smemB)) != hipSuccess)
    return fail(ZP_EHIP, "zp_score_tokens: cannot reserve %zu bytes of LDS", smemA);
  dim3 gridP(P.max_blocks, P.h_kv, items);
  hipLaunchKernelGGL(kA, gridP, dim3(256), smemA, s, P);
  if (flash) hipLaunchKernelGGL(kF, gridP, dim3(256), smemF, s, P);
  hipLaunchKernelGGL(kB, gridP, dim3(256), smemB, s, P);
  hipLaunchKernelGGL(score_finalize_kernel, dim3(P.h_kv, items), dim3(256), 0, s, P);
  return ZP_OK;
}

template <typename T, int D>
static zp_status dispatch_rows(int R, const ScoreParams& P, int items, hipStream_t s) {
  switch (R) {
    case 16: return launch_score<T, D, 16>(P, items, s);
    case 32: return launch_score<T, D, 32>(P, items, s);
    case 48: return launch_score<T, D, 48>(P, items, s);
    case 64: return launch_score<T, D, 64>(P, items, s);
    case 80: return launch_score<T, D, 80>(P, items, s);
    case 96: return launch_score<T, D, 96>(P, items, s);
    case 112: return launch_score<T, D, 112>(P, items, s);
    case 128: return launch_score<T, D, 128>(P, items, s);
    default: return fail(ZP_EINVAL, "zp_score_tokens: unsupported g*window %d", R);
  }
}

static size_t score_ws_layout(const zp_geom* g, int32_t layer_count, int32_t nreq,
                              int32_t max_blocks, size_t* stats_off, size_t* r_off,
                              size_t* s1_off, size_t* inv_off, size_t* nrm_off,
                              size_t* ksum_off, size_t* rsub_off) {
  const size_t items = size_t(layer_count) * nreq * g->num_kv_heads;
  const size_t R = size_t(group_size(g)) * g->window;
  const size_t per_tok = size_t(max_blocks) * g->block_size;
  const size_t st = kWsHeader;
  const size_t ro = round_up(st + items * max_blocks * R * 2 * sizeof(float), 256);
  const size_t so = round_up(ro + items * per_tok * sizeof(float), 256);
  const size_t io = round_up(so + items * per_tok * sizeof(float), 256);
  const size_t no = round_up(io + items * per_tok * sizeof(float), 256);
  const size_t ko = round_up(no + items * per_tok * sizeof(float), 256);
  const size_t xo = round_up(ko + items * max_blocks * g->head_dim * sizeof(float), 256);
  const size_t total = round_up(xo + items * per_tok * sizeof(unsigned long long), 256);
  if (stats_off) *stats_off = st;
  if (r_off) *r_off = ro;
  if (s1_off) *s1_off = so;
  if (inv_off) *inv_off = io;
  if (nrm_off) *nrm_off = no;
  if (ksum_off) *ksum_off = ko;
  if (rsub_off) *rsub_off = xo;
  return total;
}

}  // namespace zp

using namespace zp;

extern "C" size_t zp_score_workspace_size(const zp_geom* geom, int32_t layer_count, int32_t nreq,
                                          int32_t max_blocks) {
  if (validate_geom(geom, "zp_score_workspace_size") != ZP_OK || layer_count < 0 || nreq < 0 ||
      max_blocks < 0)
    return 0;
  return score_ws_layout(geom, layer_count, nreq, max_blocks, nullptr, nullptr, nullptr,
                         nullptr, nullptr, nullptr, nullptr);
}

extern "C" zp_status zp_score_tokens(const zp_geom* geom, const zp_cache* cache,
                                     const zp_score_params* params, int32_t layer_begin,
                                     int32_t layer_count, int32_t nreq,
                                     const int32_t* block_tables, int32_t table_stride,
                                     const int32_t* num_blocks, int32_t max_blocks,
                                     const int32_t* qslot, const uint8_t* first_compression,
                                     const uint8_t* window_lse_valid, float* scores, float* f_new,
                                     int64_t scores_stride,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  zp_status st = validate_geom(geom, "zp_score_tokens");
  if (st != ZP_OK) return st;
  if (!cache || !cache->k || !cache->qwin || !params)
    return fail(ZP_EINVAL, "zp_score_tokens: cache K / qwin or params NULL");
  if (layer_begin < 0 || layer_count < 0 || layer_begin + layer_count > geom->num_layers)
    return fail(ZP_EINVAL, "zp_score_tokens: layer range [%d, %d) outside [0, %d)", layer_begin,
                layer_begin + layer_count, geom->num_layers);
  if (nreq < 0 || max_blocks < 0 || table_stride <= 0)
    return fail(ZP_EINVAL, "zp_score_tokens: bad nreq/max_blocks/table_stride");
  if (nreq == 0 || layer_count == 0 || max_blocks == 0) return ZP_OK;
  if (!block_tables || !num_blocks || !qslot || !first_compression || !scores || !workspace)
    return fail(ZP_EINVAL, "zp_score_tokens: NULL buffer");
  if (scores_stride < int64_t(max_blocks) * geom->block_size)
    return fail(ZP_EINVAL, "zp_score_tokens: scores_stride %lld < max_blocks*b",
                (long long)scores_stride);
  const zp_score_params& sp = *params;
  if (window_lse_valid && !cache->qwin_lse)
    return fail(ZP_EINVAL, "zp_score_tokens: window_lse_valid needs cache->qwin_lse");
  if ((sp.flags & ZP_SCORE_GLOBAL) && (!cache->gscore || !f_new))
    return fail(ZP_EINVAL, "zp_score_tokens: ZP_SCORE_GLOBAL needs cache->gscore and f_new");
  if (sp.flags & ~uint32_t(ZP_SCORE_GLOBAL | ZP_SCORE_POOL | ZP_SCORE_POOL_FIRST_ONLY |
                           ZP_SCORE_REDUNDANCY | ZP_SCORE_REDUNDANCY_FLASH | ZP_SCORE_GLOBAL_SUM))
    return fail(ZP_EINVAL, "zp_score_tokens: unknown flags 0x%x", sp.flags);
  if ((sp.flags & ZP_SCORE_GLOBAL_SUM) && !(sp.flags & ZP_SCORE_GLOBAL))
    return fail(ZP_EINVAL, "zp_score_tokens: ZP_SCORE_GLOBAL_SUM needs ZP_SCORE_GLOBAL");
  if ((sp.flags & ZP_SCORE_POOL) && (sp.pool_kernel < 1 || sp.pool_kernel % 2 == 0))
    return fail(ZP_EINVAL, "zp_score_tokens: pool_kernel must be odd and >= 1");
  if ((sp.flags & ZP_SCORE_REDUNDANCY) && !(sp.tau > 0.f))
    return fail(ZP_EINVAL, "zp_score_tokens: tau must be > 0");
  if ((sp.flags & ZP_SCORE_REDUNDANCY) && !(sp.sim_threshold >= 0.f))
    return fail(ZP_EINVAL, "zp_score_tokens: sim_threshold must be >= 0");
  if (geom->max_slots <= 0) return fail(ZP_EINVAL, "zp_score_tokens: no query slots");
  size_t so, ro, s1o, io, no, ko, xo;
  const size_t need =
      score_ws_layout(geom, layer_count, nreq, max_blocks, &so, &ro, &s1o, &io, &no, &ko, &xo);
  if (workspace_bytes < need)
    return fail(ZP_EINVAL, "zp_score_tokens: workspace %zu bytes, need %zu", workspace_bytes, need);
  const int64_t items = int64_t(layer_count) * nreq;
  if (items > 65535) return fail(ZP_EINVAL, "zp_score_tokens: layer_count*nreq > 65535");

  ScoreParams P{};
  P.kc = cache->k; P.qwin = cache->qwin; P.gscore = cache->gscore;
  P.tables = block_tables; P.num_blocks = num_blocks; P.qslot = qslot;
  P.first = first_compression; P.scores = scores; P.f_new = f_new;
  P.lse_ok = window_lse_valid; P.qwin_lse = cache->qwin_lse;
  P.scores_stride = scores_stride;
  char* ws = static_cast<char*>(workspace);
  P.err = reinterpret_cast<uint32_t*>(ws);
  P.stats = reinterpret_cast<float*>(ws + so);
  P.rbuf = reinterpret_cast<float*>(ws + ro);
  P.s1buf = reinterpret_cast<float*>(ws + s1o);
  P.inv = reinterpret_cast<float*>(ws + io);
  P.nrm = reinterpret_cast<float*>(ws + no);
  P.ksum = reinterpret_cast<float*>(ws + ko);
  P.rsub = reinterpret_cast<unsigned long long*>(ws + xo);
  const int64_t d = geom->head_dim;
  P.kv_layer_elems = int64_t(geom->num_blocks) * geom->num_kv_heads * geom->block_size * d;
  P.qwin_layer_elems = int64_t(geom->max_slots) * geom->num_q_heads * geom->window * d;
  P.qlse_layer_elems = int64_t(geom->max_slots) * geom->num_q_heads * geom->window;
  P.f_layer_elems = int64_t(geom->num_blocks) * geom->num_kv_heads * geom->block_size;
  P.layer_begin = layer_begin; P.nreq = nreq; P.table_stride = table_stride;
  P.max_blocks = max_blocks; P.num_blocks_total = geom->num_blocks;
  P.b = geom->block_size; P.h_kv = geom->num_kv_heads; P.w = geom->window;
  P.max_slots = geom->max_slots;
  P.qk_scale = kLog2e / std::sqrt(float(d));
  P.alpha = sp.alpha; P.lambda_ = sp.lambda_;
  P.inv_tau = (sp.flags & ZP_SCORE_REDUNDANCY) ? 1.0f / sp.tau : 0.f;
  P.p = sp.sim_threshold; P.pool_kernel = sp.pool_kernel; P.flags = sp.flags;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int R = group_size(geom) * geom->window;
  if (geom->dtype == ZP_DTYPE_BF16) {
    st = d == 128 ? dispatch_rows<bf16_t, 128>(R, P, int(items), s)
                  : dispatch_rows<bf16_t, 64>(R, P, int(items), s);
  } else {
    st = d == 128 ? dispatch_rows<float, 128>(R, P, int(items), s)
                  : dispatch_rows<float, 64>(R, P, int(items), s);
  }
  if (st != ZP_OK) return st;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZP_EHIP, "zp_score_tokens: launch failed: %s", hipGetErrorString(e));
  return ZP_OK;
}
