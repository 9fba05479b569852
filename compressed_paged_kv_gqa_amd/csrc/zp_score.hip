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
#include <algorithm>
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
// rint(c * 2^40) from exact single-precision steps (|c| < 2^15): c * 2^16
// splits into its integer part h and a fraction in (-1, 1), which 2^24 turns
// into an integer after rounding, so the result is h * 2^24 + rint(frac * 2^24).
__device__ __forceinline__ unsigned long long to_fix(float c) {
  const float x = c * 65536.0f;
  const float h = truncf(x);
  const int lo = static_cast<int>(rintf((x - h) * 16777216.0f));
  return static_cast<unsigned long long>((static_cast<long long>(static_cast<int>(h)) << 24) + lo);
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
  if (!P.qwin_lse) return false;
  return (P.flags & ZP_SCORE_WINDOW_LSE_ALL) || (P.lse_ok && P.lse_ok[r] != 0);
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
// Flash redundancy (Zipage Alg. 3), shapes other than the serving one: one
// workgroup per column block m. Every row block i is staged in turn and its
// cosines against the columns of m are formed; each column keeps its highest row above p over the whole sequence
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
// (max, sum of exp2(x - max)) pairs merged; an empty pair is (-inf, 0).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * exp2f(m - mn) + s2 * exp2f(m2 - mn);
  m = mn;
}

template <typename T, int D, int R, bool W16>
__global__ __launch_bounds__(256, 2) void score_s0_kernel(ScoreParams P) {
  using L = LdsTile<T, D>;
  using M = Mma<T, D>;
  extern __shared__ __align__(16) char smem[];
  char* Qs = smem;                                           // [R][D]
  float* lse2 = reinterpret_cast<float*>(Qs + R * L::ROWB);  // [R]
  float* ptile = lse2 + R;                        // [4][R][16] (general window only)

  const int pidx = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
  const int r = z % P.nreq;
  if (lse_given(P, r)) return;  // done by phase A (which also flags bad geometry)
  int N, slot;
  const int page = resolve_page(P, pidx, z, &N, &slot);
  if (page < 0) return;
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
    // this window row's per-block (max, sum) pairs merged in block order,
    // four 8-byte loads in flight at a time (a loop of single loads waits
    // for each in turn)
    const float2* st = reinterpret_cast<const float2*>(P.stats + (zh * P.max_blocks) * R * 2) + tid;
    float m = -INFINITY, sm = 0.f;
    int i = 0;
    for (; i + 4 <= N; i += 4) {
      float2 a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = st[(int64_t)(i + j) * R];
#pragma unroll
      for (int j = 0; j < 4; ++j) lse_merge(m, sm, a[j].x, a[j].y);
    }
    for (; i < N; ++i) {
      const float2 a = st[(int64_t)i * R];
      lse_merge(m, sm, a.x, a.y);
    }
    lse2[tid] = m + log2f(sm);
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
// Per-request and per-block values (block counts, block ids, slots, flags)
// read through the scalar cache: the address is the same in every lane, and
// scalar loads are waited for with the LDS / scalar counter, so in the
// persistent kernels they never wait behind the in-flight HBM -> LDS copies.
typedef const __attribute__((address_space(4))) int32_t* lt_const_i32;
typedef const __attribute__((address_space(4))) uint32_t* lt_const_u32;
__device__ __forceinline__ int32_t lt_ld(const int32_t* p, int64_t i) {
  return ((lt_const_i32)p)[i];
}
__device__ __forceinline__ uint32_t lt_ld_u8(const uint8_t* p, int64_t i) {
  // the aligned word holding byte i (allocations are at least 4-byte aligned)
  const uintptr_t a = reinterpret_cast<uintptr_t>(p) + i;
  const uint32_t w = *((lt_const_u32)(a & ~uintptr_t(3)));
  return (w >> (8 * (a & 3))) & 0xffu;
}

// One workgroup of kFinThreads per (layer x request, kv-head), 4 tokens per
// thread per chunk; pooling halves up to kFinHalo are taken from an LDS copy
// of the chunk. The workgroups are all resident at once at the serving
// shapes, so the kernel takes about one workgroup's chain of dependent
// memory round trips: the request's fields are requested together, the
// block ids are checked one per thread, and the first chunk's loads (row
// sums, S1 window) all go out before the one barrier that merges the
// softmax statistics and the block-id check.
constexpr int kFinThreads = 1024, kFinChunk = 4 * kFinThreads, kFinHalo = 64;

__global__ __launch_bounds__(kFinThreads) void score_finalize_kernel(ScoreParams P) {
  constexpr int NW = kFinThreads / 64;
  __shared__ float red[2][NW];
  __shared__ int badw[NW];
  __shared__ float s1c[kFinChunk + 2 * kFinHalo];
  const int h = blockIdx.x, z = blockIdx.y;
  const int r = z % P.nreq;
  const int N = lt_ld(P.num_blocks, r);
  const int slot = lt_ld(P.qslot, r);
  const uint32_t first_w = lt_ld_u8(P.first, r);
  asm volatile("" ::"s"(N), "s"(slot), "s"(first_w));  // the three loads before any test
  if (N <= 0 || N > P.max_blocks || N > P.table_stride) return;
  if (slot < 0 || slot >= P.max_slots) return;
  const bool first = first_w != 0;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = N * P.b;  // a multiple of 16
  // A bad block id (flagged by the scoring kernels) leaves the unit's
  // scores unwritten. The ids are loaded here, one per thread, and tested
  // at the barrier below, so the loads in between are not held up.
  const int* trow = P.tables + (int64_t)r * P.table_stride;
  const int pg = tid < N ? trow[tid] : 0;
  int bad = 0;
  for (int i = tid + kFinThreads; i < N; i += kFinThreads)
    bad |= (trow[i] < 0 || trow[i] >= P.num_blocks_total) ? 1 : 0;
  const int64_t zh = (int64_t)z * P.h_kv + h;
  const float* s1 = P.s1buf + zh * ((int64_t)P.max_blocks * P.b);
  const float* rr = P.rbuf + zh * ((int64_t)P.max_blocks * P.b);
  const unsigned long long* rs = P.rsub + zh * ((int64_t)P.max_blocks * P.b);
  float* out = P.scores + zh * P.scores_stride;
  const bool pool = (P.flags & ZP_SCORE_POOL) && (first || !(P.flags & ZP_SCORE_POOL_FIRST_ONLY));
  const bool redun = (P.flags & ZP_SCORE_REDUNDANCY) != 0;
  const bool flash = redun && (P.flags & ZP_SCORE_REDUNDANCY_FLASH);
  const int half = pool ? P.pool_kernel / 2 : 0;
  const bool lds_pool = pool && half <= kFinHalo;
  const float c2 = P.inv_tau * kLog2e;  // softmax(r / tau) in the exp2 domain

  // Redundancy row values of tokens t .. t + 3; with flash redundancy the
  // row sum over the whole sequence minus its zeroed entries, / n.
  auto row4 = [&](int t) __attribute__((always_inline)) -> float4 {
    float4 x = *reinterpret_cast<const float4*>(rr + t);
    if (flash) {
      x.x = (x.x - from_fix(rs[t])) / (float)n;
      x.y = (x.y - from_fix(rs[t + 1])) / (float)n;
      x.z = (x.z - from_fix(rs[t + 2])) / (float)n;
      x.w = (x.w - from_fix(rs[t + 3])) / (float)n;
    }
    return x;
  };
  // S1 of [c0 - half, c0 + chunk + half) into s1c, -inf outside the
  // sequence: each thread its own four tokens (one 16-byte load; n is a
  // multiple of 4), the first `half` threads the halos, all loads issued
  // before any is waited for
  struct Win {
    float4 x;
    float lo, hi;
  };
  auto fill_load = [&](int c0) __attribute__((always_inline)) -> Win {
    Win f{make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY), -INFINITY, -INFINITY};
    const int t = c0 + 4 * tid;
    if (t < n) f.x = *reinterpret_cast<const float4*>(s1 + t);
    if (tid < half) {
      const int tl = c0 - half + tid, tr = c0 + kFinChunk + tid;
      if (tl >= 0) f.lo = s1[tl];
      if (tr < n) f.hi = s1[tr];
    }
    return f;
  };
  auto fill_store = [&](const Win& f) __attribute__((always_inline)) {
    float* d = s1c + half + 4 * tid;
    d[0] = f.x.x; d[1] = f.x.y; d[2] = f.x.z; d[3] = f.x.w;
    if (tid < half) {
      s1c[tid] = f.lo;
      s1c[half + kFinChunk + tid] = f.hi;
    }
  };

  // softmax statistics of r / tau in one pass: each thread's running
  // (max, sum), then the wavefront and the workgroup, in a fixed order;
  // chunk 0's row values stay in registers for the output pass
  float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f);
  float m = -INFINITY, sm = 0.f;
  Win w0{};
  if (lds_pool) w0 = fill_load(0);  // in flight with the row sums
  if (redun) {
    for (int t = 4 * tid; t < n; t += kFinChunk) {
      const float4 x = row4(t);
      if (t < kFinChunk) x0 = x;
      const float m4 = fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w)) * c2;
      const float mn = fmaxf(m, m4);
      sm = sm * exp2f(m - mn) + exp2f(x.x * c2 - mn) + exp2f(x.y * c2 - mn) +
           exp2f(x.z * c2 - mn) + exp2f(x.w * c2 - mn);
      m = mn;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lse_merge(m, sm, shfl_xor_f(m, o), shfl_xor_f(sm, o));
  }
  if (lds_pool) fill_store(w0);
  bad |= (pg < 0 || pg >= P.num_blocks_total) ? 1 : 0;
  const bool wbad = __builtin_amdgcn_ballot_w64(bad != 0) != 0;
  if (lane == 0) {
    red[0][wv] = m;
    red[1][wv] = sm;
    badw[wv] = wbad ? 1 : 0;
  }
  __syncthreads();
  int anybad = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) anybad |= badw[i];
  if (anybad) return;  // the same for every thread
  float mx = -INFINITY, inv_sum = 0.f;
  if (redun) {
    m = red[0][0];
    sm = red[1][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) lse_merge(m, sm, red[0][i], red[1][i]);
    mx = m;
    inv_sum = 1.0f / sm;
  }
  const bool vec_out = (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  for (int c0 = 0; c0 < n; c0 += kFinChunk) {
    if (lds_pool && c0 > 0) {  // chunk 0's copy was made before the barrier above
      __syncthreads();
      fill_store(fill_load(c0));
      __syncthreads();
    }
    const int t = c0 + 4 * tid;
    if (t >= n) continue;
    float v[4];
    if (lds_pool) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float mm = -INFINITY;
        for (int i = 4 * tid + e; i <= 4 * tid + e + 2 * half; ++i) mm = fmaxf(mm, s1c[i]);
        v[e] = mm;
      }
    } else if (pool) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int lo = max(0, t + e - half), hi = min(n - 1, t + e + half);
        float mm = -INFINITY;
        for (int i = lo; i <= hi; ++i) mm = fmaxf(mm, s1[i]);
        v[e] = mm;
      }
    } else {
      const float4 x = *reinterpret_cast<const float4*>(s1 + t);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    }
    if (redun) {
      const float4 x = c0 == 0 ? x0 : row4(t);
      const float xr[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] -= P.lambda_ * (exp2f(xr[e] * c2 - mx) * inv_sum);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (t + e >= n - P.w) v[e] = INFINITY;
    if (vec_out) {
      *reinterpret_cast<float4*>(out + t) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) out[t + e] = v[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Phase A, persistent form for the serving shape (bf16, head_dim 128, blocks
// of 256 tokens, a 16-token window, g <= 4 query heads per kv-head): one
// workgroup of 16 wavefronts per CU walks a
// contiguous range of the (layer, kv-head, request, block) items. The next
// item's keys, global-score history and window log-sum-exp are copied
// HBM -> LDS (global_load_lds, no registers) into the second of two buffers
// while the current item is scored, so the copy of every block after the
// first overlaps the work on the one before. Items run in the order
// (layer, kv-head, request, block), so consecutive items of a workgroup
// share their window queries, which are copied only when the request or
// kv-head changes. Per item:
//   1. MFMA window logits of the wave's column tile against the g*16 window
//      rows (LDS), giving S0 and the global score from the window
//      log-sum-exp, or each row's partial (max, sum); key norms, four lanes
//      per key;
//   2. MFMA cosine tiles: wave w takes 2 column tiles against 8 of the 16
//      row tiles and keeps, per column, the sum of k_i . k_j / |k_i| over
//      its rows and the highest row whose cosine is above p (the Gram
//      matrix is symmetric, so a column's sum is the row sum of the same
//      key);
//   3. per column, the two halves combined and its zeroed entry (one dot
//      product) added to that entry's row in 64-bit fixed point (exact, so
//      the same bits in any order);
//   4. each row's sum minus its zeroed entries, / n: the redundancy row
//      sums (made at the start of the next item, so that no barrier of its
//      own is needed).
// With flash redundancy, steps 2-4 belong to score_flash_persist_kernel: the
// item writes its key norms for it and clears its fixed-point words.
// ---------------------------------------------------------------------------
// Barrier over LDS traffic only: each wavefront's LDS operations are
// complete (lgkmcnt 0), its HBM loads and copies into LDS are not waited for.
// A __syncthreads() (whose fence also waits for copies into LDS) would wait
// for the next item's copies, which are meant to stay in flight; the LDS
// they fill is read only after the full wait at the end of the item. The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt and expcnt at their maximum, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Max over lane pairs (l, l ^ 16) / (l, l ^ 32) of an int, with the row swaps.
__device__ __forceinline__ int xor16_max_i(int v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max((int)r[0], (int)r[1]);
}
// IEEE maximum (gfx950 v_maximum3_f32): fmaxf must first quiet inputs the
// compiler cannot prove canonical (MFMA results, LDS loads, DPP moves), one
// v_max_f32 each; this needs none. The values it sees carry no NaN unless
// the inputs do (masked logits are -inf by selection).
__device__ __forceinline__ float max_nq(float a, float b) { return __builtin_elementwise_maximum(a, b); }
template <int LANES>
__device__ __forceinline__ float group_max_nq(float v) {
  static_assert(LANES == 16, "16-lane rows");
  v = max_nq(v, dpp_f<DPP_QUAD_XOR1>(v));
  v = max_nq(v, dpp_f<DPP_QUAD_XOR2>(v));
  v = max_nq(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  return max_nq(v, dpp_f<DPP_ROW_MIRROR>(v));
}
// IEEE maximum over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_max_nq(float v) {
  v = group_max_nq<16>(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max_nq(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_nq(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}
// Per column, the largest raw product of a tile above which an entry
// k_i . k_j / |k_i| of it may exceed p |k_j| (pnc): pnc / (the largest 1/|k_i|
// over the rows, ivx), less 1e-5 relative so that rounding can only let more
// tiles through to the exact test (an entry above pnc >= 0 has a positive
// product, and product * 1/|k_i| <= largest product * ivx). ivx = 0 (no
// norm) gives +inf (no entry can pass), pnc = 0 with it NaN (every tile
// passes to the exact test).
__device__ __forceinline__ float product_threshold(float pnc, float ivx) {
  return pnc * __builtin_amdgcn_rcpf(ivx) * (1.0f - 1.0e-5f);
}

__device__ __forceinline__ int xor32_max_i(int v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((int)r[0], (int)r[1]);
}

// 64-bit add to an LDS word, no return value. Written as the instruction
// itself: the compiler would otherwise wait for every copy into LDS still in
// flight (vmcnt 0) before an LDS atomic, whatever its address; this one
// touches only `sub`, which no copy writes. lds_barrier()'s lgkmcnt wait
// completes it.
__device__ __forceinline__ void lds_add_u64(unsigned long long* p, unsigned long long v) {
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned long long*)p;
  asm volatile("ds_add_u64 %0, %1" ::"v"(a), "v"(v) : "memory");
}

typedef __attribute__((address_space(3))) void* lt_lds_ptr;
typedef __attribute__((address_space(1))) void* lt_gbl_ptr;

constexpr int kLtThreads = 1024;

// Cursor over the items of one workgroup, with the values its item needs.
struct LtItem {
  int li, h, r, pidx, N;  // layer index in the call, kv-head, request, block, blocks of r
  int page, slot;
  bool valid, first, lse;
};

// Blocks of request r that scoring covers (0 when its geometry is invalid;
// such a request is flagged once by workgroup 0).
__device__ __forceinline__ int lt_blocks(const ScoreParams& P, int r) {
  const int N = lt_ld(P.num_blocks, r);
  return (N <= 0 || N > P.max_blocks || N > P.table_stride) ? 0 : N;
}

__device__ __forceinline__ void lt_fill(const ScoreParams& P, LtItem& it) {
  // four independent loads, no branch between them (one wait): without a
  // window-LSE flag array the first-flag word is read in its place and
  // ignored
  const uint8_t* lp = P.lse_ok ? P.lse_ok : P.first;
  const int32_t page = lt_ld(P.tables, (int64_t)it.r * P.table_stride + it.pidx);
  const int32_t slot = lt_ld(P.qslot, it.r);
  const uint32_t f = lt_ld_u8(P.first, it.r);
  const uint32_t l = lt_ld_u8(lp, it.r);
  it.page = page;
  it.slot = slot;
  it.first = f != 0;
  it.lse = P.qwin_lse != nullptr &&
           ((P.flags & ZP_SCORE_WINDOW_LSE_ALL) || (P.lse_ok != nullptr && l != 0));
}

__device__ __forceinline__ void lt_next_request(const ScoreParams& P, LtItem& it, int layer_count) {
  // first request (at or after it.r) with blocks, moving to the next kv-head
  // and layer as needed
  for (;;) {
    if (it.r >= P.nreq) {
      it.r = 0;
      if (++it.h >= P.h_kv) {
        it.h = 0;
        if (++it.li >= layer_count) {
          it.valid = false;
          return;
        }
      }
    }
    it.N = lt_blocks(P, it.r);
    if (it.N > 0) return;
    ++it.r;
  }
}

// Moves the cursor k >= 1 items on (the next item is k = 1), then loads
// the new item's block id, slot and flags once.
__device__ __forceinline__ void lt_skip(const ScoreParams& P, LtItem& it, int k, int layer_count) {
  for (;;) {
    const int room = it.N - 1 - it.pidx;  // items after this one in the same request
    if (k <= room) {
      it.pidx += k;
      break;
    }
    k -= room + 1;
    it.pidx = 0;
    ++it.r;
    lt_next_request(P, it, layer_count);
    if (!it.valid) return;
  }
  lt_fill(P, it);
}
// Moves the cursor to the next item. `next_page` holds the block id after
// the current item in its request, read by the previous call (an item
// ahead, so its wait falls behind that item's work); the call reads the one
// after the new item the same way (the index is clamped to the request's
// last block, whose id is then not used).
__device__ __forceinline__ void lt_advance(const ScoreParams& P, LtItem& it, int layer_count,
                                           int& next_page) {
  if (++it.pidx >= it.N) {
    it.pidx = 0;
    ++it.r;
    lt_next_request(P, it, layer_count);
    if (it.valid) lt_fill(P, it);
  } else {  // same request: only the block id changes
    it.page = next_page;
  }
  if (it.valid)
    next_page = lt_ld(P.tables, (int64_t)it.r * P.table_stride + min(it.pidx + 1, it.N - 1));
}

// Blocks of request r, one request per lane, read with a vector load: every
// lane's load is in flight at once (0 past the last request and for a
// request whose geometry is invalid, which `flag` reports).
__device__ __forceinline__ int lt_lane_blocks(const ScoreParams& P, int r, bool flag) {
  int N = 0;
  if (r < P.nreq) {
    N = P.num_blocks[r];
    if (N > P.max_blocks || N > P.table_stride) {
      if (flag) flag_error(P.err, ZP_DEVERR_SEQ_LEN);
      N = 0;
    } else if (N < 0) {
      N = 0;
    }
  }
  return N;
}

// Inclusive prefix sum over the 64 lanes of the wavefront.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// The call's valid blocks over all requests, 64 requests per step (the
// same value in every wavefront).
__device__ __forceinline__ int lt_total_blocks(const ScoreParams& P, bool flag) {
  int S = 0;
  for (int r0 = 0; r0 < P.nreq; r0 += 64) {
    const int inc = wave_incl_scan(lt_lane_blocks(P, r0 + (threadIdx.x & 63), flag));
    S += __builtin_amdgcn_readlane(inc, 63);
  }
  return S;
}

// Places the cursor on the call's valid block s (0 <= s < the total): the
// first request whose running block count exceeds s, found with a prefix
// sum and a ballot over 64 requests per step. False if s is past the end.
__device__ __forceinline__ bool lt_locate(const ScoreParams& P, int s, LtItem& it) {
  for (int r0 = 0; r0 < P.nreq; r0 += 64) {
    const int N = lt_lane_blocks(P, r0 + (threadIdx.x & 63), false);
    const int inc = wave_incl_scan(N);
    const unsigned long long hit = __ballot(inc > s);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      it.r = r0 + l;
      it.N = __builtin_amdgcn_readlane(N, l);
      it.pidx = s - (__builtin_amdgcn_readlane(inc, l) - it.N);
      return true;
    }
    s -= __builtin_amdgcn_readlane(inc, 63);
  }
  return false;
}

template <int RT>
__global__ __launch_bounds__(kLtThreads, 1) void score_lightning_kernel(ScoreParams P,
                                                                       int layer_count) {
  constexpr int R = RT * 16;  // window rows: g query heads x 16 window slots
  constexpr int D = 128, BT = 256;
  using L = LdsTile<bf16_t, D>;
  using M = Mma<bf16_t, D>;
  __shared__ __align__(16) char Ka[BT * L::ROWB];
  __shared__ __align__(16) char Kb[BT * L::ROWB];
  __shared__ __align__(16) char Qs[R * L::ROWB];
  __shared__ __align__(16) float Fa[BT];
  __shared__ __align__(16) float Fb[BT];
  __shared__ __align__(16) float La[R];
  __shared__ __align__(16) float Lb[R];
  __shared__ __align__(16) float inv_s[BT];
  __shared__ __align__(16) float nrm_s[BT];
  __shared__ __align__(16) unsigned long long sub[BT];
  __shared__ __align__(16) float csum[2][BT];  // per half of the rows: the column's sum (then csum[0]: the row sum),
  __shared__ __align__(16) short crow[2][BT];  //   the highest row above p (-1: none)
  __shared__ __align__(16) float wstat[8][R][2];  // window-row statistics (waves 0..7)

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const bool redun = (P.flags & ZP_SCORE_REDUNDANCY) != 0;
  const bool flash = redun && (P.flags & ZP_SCORE_REDUNDANCY_FLASH) != 0;
  const bool glob = (P.flags & ZP_SCORE_GLOBAL) != 0;
  const float sc2 = P.qk_scale;

  // The workgroup's range of items, in units of the call's valid blocks.
  const int S = lt_total_blocks(P, blockIdx.x == 0 && wv == 0);
  const int64_t V = (int64_t)layer_count * P.h_kv * S;
  const int64_t v0 = V * blockIdx.x / gridDim.x, v1 = V * (blockIdx.x + 1) / gridDim.x;
  if (v0 >= v1) return;
  LtItem cur;
  {
    cur.li = (int)(v0 / ((int64_t)P.h_kv * S));
    const int64_t rem = v0 % ((int64_t)P.h_kv * S);
    cur.h = (int)(rem / S);
    cur.valid = true;
    if (!lt_locate(P, (int)(rem % S), cur)) return;
    lt_fill(P, cur);
  }
  int left = (int)(v1 - v0);  // items this workgroup still scores, the current one included

  // The item loop reads the call's parameters through `pq`, the kernel
  // argument segment (P is its first argument, at offset 0), re-read from
  // an opaque copy of its address at each item. The compiler then reloads a
  // field with a scalar load where the item uses it, instead of holding ~60
  // parameter registers across the item's straight-line body and spilling
  // them to VGPR lanes (84 spilled SGPRs, ~200 `v_readlane` per item, before).
  typedef const __attribute__((address_space(4))) ScoreParams* kp_t;
  const kp_t kp0 = (kp_t)__builtin_amdgcn_kernarg_segment_ptr();
  const ScoreParams* pq = (const ScoreParams*)kp0;
  auto relaunder = [&]() __attribute__((always_inline)) {
    uint64_t u = (uint64_t)kp0;
    asm volatile("" : "+s"(u));
    pq = (const ScoreParams*)(kp_t)u;
  };
  auto item_ok = [&](const LtItem& it) -> bool {
    return it.page >= 0 && it.page < pq->num_blocks_total && it.slot >= 0 && it.slot < pq->max_slots;
  };

  // Copies item `it`'s keys (swizzled tile), history F and window LSE into
  // (Kd, Fd, Ld): every wavefront 4 KiB of keys; wavefront 0 F, wavefront 1
  // the LSE.
  auto issue = [&](const LtItem& it, char* Kd, float* Fd, float* Ld) __attribute__((always_inline)) {
    if (!item_ok(it)) return;
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));  // per item: keeps the addresses out of the loop
    const int layer = pq->layer_begin + it.li;
    const char* kp = reinterpret_cast<const char*>(
        reinterpret_cast<const bf16_t*>(pq->kc) + layer * pq->kv_layer_elems +
        ((int64_t)it.page * pq->h_kv + it.h) * BT * D);
    // Byte offsets, inside the block, of the four 16-byte chunks this lane
    // copies: LDS chunk p = (4 wv + i) 64 + lane of the swizzled tile holds
    // row p / 16 = 16 wv + 4 i + lane / 16 and chunk (p % 16) ^ (row % 16)
    // = (lane % 16) ^ (lane / 16) ^ 4 i, so chunk i sits at
    // kb + 1024 i + (kc ^ 64 i).
    const int kb = (16 * wv + (lane >> 4)) * L::ROWB, kc = ((lane & 15) ^ (lane >> 4)) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds((lt_gbl_ptr)(kp + kb + 1024 * i + (kc ^ (64 * i))),
                                       (lt_lds_ptr)(Kd + (wv * 4 + i) * 1024), 16, 0, 0);
    if (glob && !it.first && wv == 0) {  // 1 KiB, 16 bytes per lane
      const float* fp = pq->gscore + layer * pq->f_layer_elems + ((int64_t)it.page * pq->h_kv + it.h) * BT;
      __builtin_amdgcn_global_load_lds((lt_gbl_ptr)(fp + lane * 4), (lt_lds_ptr)Fd, 16, 0, 0);
    }
    if (wv == 1 && it.lse && lane < R / 4) {  // R floats, 16 bytes per lane
      const float* lp = pq->qwin_lse + layer * pq->qlse_layer_elems + ((int64_t)it.slot * pq->h_kv + it.h) * R;
      __builtin_amdgcn_global_load_lds((lt_gbl_ptr)(lp + lane * 4), (lt_lds_ptr)Ld, 16, 0, 0);
    }
  };
  // The window queries of item `it` into Qs (R rows, swizzled like K):
  // R / 4 copies of 1 KiB, one per wavefront.
  auto issue_q = [&](const LtItem& it) __attribute__((always_inline)) {
    if (it.slot < 0 || it.slot >= pq->max_slots || wv >= R / 4) return;
    const int layer = pq->layer_begin + it.li;
    const char* qp = reinterpret_cast<const char*>(
        reinterpret_cast<const bf16_t*>(pq->qwin) + layer * pq->qwin_layer_elems +
        ((int64_t)it.slot * pq->h_kv + it.h) * R * D);
    const int p = wv * 64 + lane;
    const int rr = p >> 4, c = (p & 15) ^ (rr & 15);
    __builtin_amdgcn_global_load_lds((lt_gbl_ptr)(qp + rr * L::ROWB + c * 16),
                                     (lt_lds_ptr)(Qs + wv * 1024), 16, 0, 0);
  };

  // 4. of the previous item, row i: (row sum - zeroed entries) / n, and its
  // fixed-point word cleared. Run before this item's first barrier: csum
  // and sub are written again only after it, and the barrier that ended
  // the previous item retired its LDS adds.
  bool pend = false;
  int64_t pend_off = 0;
  float pend_n = 1.f;
  auto flush_rows = [&](int t) __attribute__((always_inline)) {
    if (pend && t < BT) {
      pq->rbuf[pend_off + t] = (csum[0][t] - from_fix(sub[t])) / pend_n;
      sub[t] = 0ull;
    }
    pend = false;
  };

  // Scores item `it` from (Kt, Ft, Lt); `nx` is the next item (its queries
  // are copied into Qs once this item's window phase is done).
  auto process = [&](const LtItem& it, const LtItem& nx, const char* Kt, const float* Ft,
                     const float* Lt) __attribute__((always_inline)) {
    // Thread ids laundered once per item: the compiler would otherwise hoist
    // every lane-dependent LDS address out of the item loop and keep them
    // all live (register spills).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, q = lane >> 4, cl = lane & 15;
    flush_rows(tid);
    const bool ok = item_ok(it);
    const int z = it.li * pq->nreq + it.r;
    const int64_t zh = (int64_t)z * pq->h_kv + it.h;
    const bool last = it.pidx == it.N - 1;
    const int n = it.N * BT;
    if (!ok && tid == 0) {
      flag_error(pq->err, (it.page < 0 || it.page >= pq->num_blocks_total) ? ZP_DEVERR_BLOCK_ID
                                                                        : ZP_DEVERR_SLOT);
    }
    // 1. window logits (LSE given: wave w takes column tile w; statistics:
    // waves 0..7 take column tiles w, w + 8) and key norms (4 lanes per key)
    if (ok) {
      if (it.lse) {
        typename M::op_t bop[M::NKS];
#pragma unroll
        for (int ks = 0; ks < M::NKS; ++ks) bop[ks] = M::lds(Kt, wv * 16 + cl, ks, lane);
        // the group max of P = exp2(logit - lse) is exp2 of the group max
        // of (logit - lse): one exp2 per window slot
        float pm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        __builtin_amdgcn_s_setprio(3);  // stepped down per row tile, as in the cosine phase
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          if (rt == 1) __builtin_amdgcn_s_setprio(2);
          if (rt == 2) __builtin_amdgcn_s_setprio(1);
          if (rt == 3) __builtin_amdgcn_s_setprio(0);
          typename M::op_t a[M::NKS];
#pragma unroll
          for (int ks = 0; ks < M::NKS; ++ks) a[ks] = M::lds(Qs, rt * 16 + cl, ks, lane);
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < M::NKS; ++ks) acc = M::mma(a[ks], bop[ks], acc);
          const float4 l4 = *reinterpret_cast<const float4*>(Lt + rt * 16 + 4 * q);
          const float lv[4] = {l4.x * kLog2e, l4.y * kLog2e, l4.z * kLog2e, l4.w * kLog2e};
#pragma unroll
          for (int v = 0; v < 4; ++v) pm[v] = max_nq(pm[v], fmaf(acc[v], sc2, -lv[v]));
        }
        __builtin_amdgcn_s_setprio(0);
        const int col = wv * 16 + cl;
        if (redun) {
          // |k|^2 of the wavefront's 16 keys from its operand registers:
          // lanes cl, cl + 16, cl + 32, cl + 48 hold the 128 dimensions of
          // key cl (no second LDS pass over the block)
          typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
          float ss = 0.f;
#pragma unroll
          for (int ks = 0; ks < M::NKS; ++ks) {
            const uint4 u = __builtin_bit_cast(uint4, bop[ks]);
            ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.x), __builtin_bit_cast(bf2, u.x), ss, false);
            ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.y), __builtin_bit_cast(bf2, u.y), ss, false);
            ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.z), __builtin_bit_cast(bf2, u.z), ss, false);
            ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.w), __builtin_bit_cast(bf2, u.w), ss, false);
          }
          ss = xor32_sum(xor16_sum(ss));
          if (q == 0) {
            const float nr = sqrtf(ss);
            inv_s[col] = ss > 0.f ? __builtin_amdgcn_rcpf(nr) : 0.f;  // v_rcp_f32, 1 ulp
            nrm_s[col] = nr;
          }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) pm[v] = __builtin_amdgcn_exp2f(pm[v]);
        if (last) {  // causal mask: window slot u = 4q + v sees keys up to BT - 16 + u
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (col > BT - 16 + 4 * q + v) pm[v] = 0.f;
        }
        float s = (pm[0] + pm[1]) + (pm[2] + pm[3]);
        s = xor32_sum(xor16_sum(s));
        if (q == 0) {
          const float s0 = s * (1.0f / 16.0f);
          float s1 = s0;
          if (glob) {
            if (!it.first && !last) {
              const float f = pq->alpha * Ft[col];
              s1 = (pq->flags & ZP_SCORE_GLOBAL_SUM) ? f + s0 : fmaxf(f, s0);
            }
            pq->f_new[zh * pq->scores_stride + (int64_t)it.pidx * BT + col] = s1;
          }
          pq->s1buf[zh * ((int64_t)pq->max_blocks * BT) + (int64_t)it.pidx * BT + col] = s1;
        }
      } else if (wv < 8) {
        // partial (max, sum of exp2) of each row over this wave's 32 columns
        typename M::op_t bop[2][M::NKS];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int ks = 0; ks < M::NKS; ++ks) bop[c][ks] = M::lds(Kt, (wv + 8 * c) * 16 + cl, ks, lane);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          typename M::op_t a[M::NKS];
#pragma unroll
          for (int ks = 0; ks < M::NKS; ++ks) a[ks] = M::lds(Qs, rt * 16 + cl, ks, lane);
          floatx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
          for (int ks = 0; ks < M::NKS; ++ks)
#pragma unroll
            for (int c = 0; c < 2; ++c) acc[c] = M::mma(a[ks], bop[c][ks], acc[c]);
          if (last) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
              for (int v = 0; v < 4; ++v)
                if ((wv + 8 * c) * 16 + cl > BT - 16 + 4 * q + v) acc[c][v] = -INFINITY;
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float Mx = group_max_nq<16>(max_nq(acc[0][v], acc[1][v]));
            const float ms = Mx == -INFINITY ? 0.f : Mx * sc2;
            float sm = __builtin_amdgcn_exp2f(fmaf(acc[0][v], sc2, -ms)) +
                       __builtin_amdgcn_exp2f(fmaf(acc[1][v], sc2, -ms));
            sm = group_sum<16>(sm);
            if (cl == 0) {
              wstat[wv][rt * 16 + 4 * q + v][0] = Mx == -INFINITY ? -INFINITY : ms;
              wstat[wv][rt * 16 + 4 * q + v][1] = sm;
            }
          }
        }
      }
      if (redun && !it.lse) {  // |k|^2, 4 lanes per key (32 dimensions each)
        const int row = tid >> 2, part = tid & 3;
        float ss = 0.f;
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int c = part * 4; c < part * 4 + 4; ++c) {
          const uint4 u = *reinterpret_cast<const uint4*>(Kt + L::chunk_pos(row, c) * 16);
          ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.x), __builtin_bit_cast(bf2, u.x), ss, false);
          ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.y), __builtin_bit_cast(bf2, u.y), ss, false);
          ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.z), __builtin_bit_cast(bf2, u.z), ss, false);
          ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.w), __builtin_bit_cast(bf2, u.w), ss, false);
        }
        ss += dpp_f<DPP_QUAD_XOR1>(ss);
        ss += dpp_f<DPP_QUAD_XOR2>(ss);
        if (part == 0) {
          const float nr = sqrtf(ss);
          inv_s[row] = ss > 0.f ? __builtin_amdgcn_rcpf(nr) : 0.f;  // v_rcp_f32, 1 ulp
          nrm_s[row] = nr;
        }
      }
    }
    lds_barrier();  // B1: norms and window rows done; Qs free
    if (nx.valid && (nx.li != it.li || nx.h != it.h || nx.r != it.r)) issue_q(nx);
    if (ok && !it.lse && tid < R) {
      float Mx = -INFINITY;
#pragma unroll
      for (int w2 = 0; w2 < 8; ++w2) Mx = max_nq(Mx, wstat[w2][tid][0]);
      float Sm = 0.f;
      if (Mx != -INFINITY)
#pragma unroll
        for (int w2 = 0; w2 < 8; ++w2) Sm += wstat[w2][tid][1] * exp2f(wstat[w2][tid][0] - Mx);
      float* st = pq->stats + ((zh * pq->max_blocks + it.pidx) * R + tid) * 2;
      st[0] = Mx;
      st[1] = Sm;
    }
    if (ok && flash) {  // flash: the norms for its own kernel, its fixed-point words cleared
      if (tid < BT) {
        const int64_t o = zh * ((int64_t)pq->max_blocks * BT) + (int64_t)it.pidx * BT + tid;
        pq->inv[o] = inv_s[tid];
        pq->nrm[o] = nrm_s[tid];
        pq->rsub[o] = 0ull;
      }
      return;
    }
    if (!ok || !redun) return;
    // 2. cosine tiles: wave w takes column tiles 2(w % 8), +1 against row
    // tiles 8(w / 8) .. +7. Per column, over the wave's rows: the highest
    // row whose entry is above p, and the sum of the entries,
    // sum_i k_i . k_j / |k_i|, the diagonal left out. The matrix is
    // symmetric, so column j's sum is row j's. Software-pipelined: the
    // products of row tile k + 1 are issued before the epilogue of tile k.
    {
      const int cg = wv & 7, rh = wv >> 3;
      const int kd = 2 * cg - 8 * rh;  // local row tile of the diagonal tile of c = 0, if in range
      const bool has_diag = (cg >> 2) == rh;
      typename M::op_t bop[2][M::NKS];
      float pnc[2], cs[2] = {0.f, 0.f};
      int bk[2] = {-1, -1};  // 4 * local row tile + v of the highest entry above p
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int ks = 0; ks < M::NKS; ++ks) bop[c][ks] = M::lds(Kt, (2 * cg + c) * 16 + cl, ks, lane);
        pnc[c] = pq->p * nrm_s[(2 * cg + c) * 16 + cl];
      }
      bool dg[4];  // this lane's element on the diagonal of a diagonal tile
#pragma unroll
      for (int v = 0; v < 4; ++v) dg[v] = 4 * q + v == cl;
      // this half's rows (row tile 8 rh + k is row tile k from here: the
      // swizzle depends on the row only modulo 16, so each tile's addresses
      // are the first's plus a constant)
      const char* Kh = Kt + rh * 128 * L::ROWB;
      const float* ivh = inv_s + rh * 128;
      const float ivx = wave_max_nq(max_nq(ivh[lane], ivh[lane + 64]));  // over this half's rows
      const float thr[2] = {product_threshold(pnc[0], ivx), product_threshold(pnc[1], ivx)};
      // Software-pipelined two deep: in step k the operands of tile k + 2
      // and the inverse norms of tile k + 1 are read from LDS, tile k + 1's
      // products are issued, and tile k's epilogue runs, so no step waits
      // on an LDS read or a product issued in the same step.
      auto load_a = [&](int k, typename M::op_t* a) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < M::NKS; ++ks) a[ks] = M::lds(Kh, k * 16 + cl, ks, lane);
      };
      auto products = [&](const typename M::op_t* a, floatx4* acc) __attribute__((always_inline)) {
        acc[0] = floatx4{0.f, 0.f, 0.f, 0.f};
        acc[1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < M::NKS; ++ks)
#pragma unroll
          for (int c = 0; c < 2; ++c) acc[c] = M::mma(a[ks], bop[c][ks], acc[c]);
      };
      typename M::op_t aA[M::NKS], aB[M::NKS];
      floatx4 accA[2], accB[2];
      float4 ivA, ivB;
      // The four wavefronts of a SIMD would otherwise finish this phase
      // apart (the oldest issues first) and wait for the last at the next
      // barrier: a wavefront's priority steps down as its tiles are done,
      // so the ones behind get the issue slots.
      __builtin_amdgcn_s_setprio(3);
      load_a(0, aA);
      load_a(1, aB);
      ivA = *reinterpret_cast<const float4*>(ivh + 4 * q);
      products(aA, accA);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k == 2) __builtin_amdgcn_s_setprio(2);
        if (k == 4) __builtin_amdgcn_s_setprio(1);
        if (k == 6) __builtin_amdgcn_s_setprio(0);
        floatx4* cur = (k & 1) ? accB : accA;
        floatx4* nxt = (k & 1) ? accA : accB;
        typename M::op_t* an = (k & 1) ? aA : aB;  // operands of tile k + 1
        typename M::op_t* af = (k & 1) ? aB : aA;  // free: tile k's, consumed last step
        const float4 iv = (k & 1) ? ivB : ivA;
        if (k < 6) load_a(k + 2, af);
        if (k < 7) {
          float4& ivn = (k & 1) ? ivA : ivB;
          ivn = *reinterpret_cast<const float4*>(ivh + (k + 1) * 16 + 4 * q);
          products(an, nxt);
        }
        const float ivv[4] = {iv.x, iv.y, iv.z, iv.w};
        // x = k_i . k_j / |k_i| is summed for the column (the diagonal, k_j
        // against itself, is taken out after the loop), and is above p |k_j|
        // exactly when the cosine is above p
        float cmx[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          cs[c] = fmaf(cur[c][3], ivv[3], fmaf(cur[c][2], ivv[2], fmaf(cur[c][1], ivv[1], fmaf(cur[c][0], ivv[0], cs[c]))));
          cmx[c] = max_nq(max_nq(cur[c][0], cur[c][1]), max_nq(cur[c][2], cur[c][3]));
        }
        // the highest row above p, tracked only in tiles that have one (the
        // test is made for the whole wavefront at once; a diagonal tile
        // always has one, its diagonal, which is never the entry to zero):
        // a tile whose largest product per column stays at or below that
        // column's threshold has none; NaN passes to the exact test
        const bool any = !(cmx[0] <= thr[0]) || !(cmx[1] <= thr[1]);
        if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const bool isd = has_diag && k == kd + c;  // wave-uniform
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const bool hit = cur[c][v] * ivv[v] > pnc[c] && !(isd && dg[v]);
              bk[c] = hit ? 4 * k + v : bk[c];
            }
          }
        }
        // the epilogue of tile k is made here (not deferred, which would
        // keep every tile's products live); tile k + 1's products overlap it
#pragma unroll
        for (int c = 0; c < 2; ++c) asm volatile("" : "+v"(bk[c]), "+v"(cs[c]));
        __builtin_amdgcn_sched_barrier(0);
      }
      // over the four row groups q of the 16 lanes of each column: the
      // highest row and the sum, in a fixed order
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = bk[c] < 0 ? -1 : (8 * rh + (bk[c] >> 2)) * 16 + 4 * q + (bk[c] & 3);
        const int top = xor32_max_i(xor16_max_i(row));
        const int col = (2 * cg + c) * 16 + cl;
        float sum = xor32_sum(xor16_sum(cs[c]));
        // the diagonal entry k_j . k_j / |k_j| = |k_j| out of the sum
        if (has_diag) sum -= nrm_s[col];
        if (q == 0) {
          crow[rh][col] = (short)top;
          csum[rh][col] = sum;
        }
      }
    }
    lds_barrier();  // B2
    // 3. per column j (four threads, 32 dimensions each): its row sum, and
    // its zeroed entry (the highest row above p over both halves), added to
    // that row in 64-bit fixed point (the same bits in any order)
    {
      const int j = tid >> 2, part = tid & 3;
      const int r1 = crow[1][j];
      const int is = r1 >= 0 ? r1 : (int)crow[0][j];  // rows of half 1 are the higher ones
      float d = 0.f;
      if (is >= 0) {
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int c = part * 4; c < part * 4 + 4; ++c) {
          const uint4 u = *reinterpret_cast<const uint4*>(Kt + L::chunk_pos(is, c) * 16);
          const uint4 w = *reinterpret_cast<const uint4*>(Kt + L::chunk_pos(j, c) * 16);
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.x), __builtin_bit_cast(bf2, w.x), d, false);
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.y), __builtin_bit_cast(bf2, w.y), d, false);
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.z), __builtin_bit_cast(bf2, w.z), d, false);
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.w), __builtin_bit_cast(bf2, w.w), d, false);
        }
      }
      d += dpp_f<DPP_QUAD_XOR1>(d);
      d += dpp_f<DPP_QUAD_XOR2>(d);
      if (part == 0) {
        const float ivj = inv_s[j];
        csum[0][j] = (csum[0][j] + csum[1][j]) * ivj;
        if (is >= 0) lds_add_u64(&sub[is], to_fix(d * inv_s[is] * ivj));
      }
    }
    // 4. is left to the start of the next item (or the end of the loop),
    // after the barrier that ends this one
    pend = true;
    pend_off = zh * ((int64_t)pq->max_blocks * BT) + (int64_t)it.pidx * BT;
    pend_n = (float)n;
  };

  if (tid < BT) sub[tid] = 0ull;
  int next_page = lt_ld(pq->tables, (int64_t)cur.r * pq->table_stride + min(cur.pidx + 1, cur.N - 1));
  issue(cur, Ka, Fa, La);
  issue_q(cur);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (;;) {
    relaunder();
    LtItem nx = cur;
    if (left > 1) lt_advance(*pq, nx, layer_count, next_page); else nx.valid = false;
    if (nx.valid) issue(nx, Kb, Fb, Lb);
    process(cur, nx, Ka, Fa, La);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (!nx.valid) break;
    cur = nx;
    --left;
    relaunder();
    nx = cur;
    if (left > 1) lt_advance(*pq, nx, layer_count, next_page); else nx.valid = false;
    if (nx.valid) issue(nx, Ka, Fa, La);
    process(cur, nx, Kb, Fb, Lb);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (!nx.valid) break;
    cur = nx;
    --left;
  }
  flush_rows(tid);
}

// ---------------------------------------------------------------------------
// Flash redundancy, persistent form for the serving shape (bf16, head_dim
// 128, blocks of 256): one workgroup of 16 wavefronts per CU walks a
// contiguous range of (layer, kv-head, request, column block m) items. The
// column block's MFMA operands are read once per item into registers (wave
// w: column tiles 2(w % 8), +1); the request's row blocks i = 0 .. N - 1
// stream through two LDS buffers (keys and their inverse norms, copied
// HBM -> LDS with global_load_lds while the previous row block is used;
// the copy of the next item's first row block overlaps the current item's
// last). Per row block the wavefront forms the cosine tiles of its 8 row
// tiles (half w / 8 of the block) against its 2 column tiles, exactly as
// the lightning kernel does, and keeps per column, over the whole sequence:
// the sum of k_i . k_j / |k_i| and the highest row whose cosine is above p
// (rows run in ascending order, so the last hit is the highest). The
// diagonal (block m against itself) is left out. At the end of the item,
// per column j: the row sum of cosines of key j (the matrix is symmetric),
// and its zeroed entry added to that entry's row in 64-bit fixed point
// (global atomics: other items hold other columns of the same rows; exact,
// so the same bits in any order). The score finalize subtracts them.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kLtThreads, 1) void score_flash_persist_kernel(ScoreParams P,
                                                                           int layer_count) {
  constexpr int D = 128, BT = 256;
  using L = LdsTile<bf16_t, D>;
  using M = Mma<bf16_t, D>;
  __shared__ __align__(16) char Ka[BT * L::ROWB];
  __shared__ __align__(16) char Kb[BT * L::ROWB];
  __shared__ __align__(16) float Ia[BT];
  __shared__ __align__(16) float Ib[BT];
  __shared__ __align__(16) float csum[2][BT];  // per half of the rows: the column's sum,
  __shared__ __align__(16) int crow[2][BT];    //   the highest row above p (-1: none)

  const int wv = wave_id();
  const int S = lt_total_blocks(P, false);
  // Items (layer, kv-head, request, column block) in order, a unit's column
  // blocks adjacent. Workgroups reach the 8 XCDs round-robin; each XCD gets
  // a contiguous share of the items, which its Gx workgroups take in stride,
  // so at any time they work on the column blocks of one or two units and
  // the row blocks every column block streams come from that XCD's L2.
  const int64_t V = (int64_t)layer_count * P.h_kv * S;
  const int G = gridDim.x, xcd = blockIdx.x & 7, l8 = blockIdx.x >> 3;
  const int g8 = G >> 3, gr = G & 7;
  const int cw0 = xcd * g8 + min(xcd, gr), cw1 = (xcd + 1) * g8 + min(xcd + 1, gr);
  const int Gx = cw1 - cw0;  // workgroups on this XCD, l8 < Gx
  const int64_t xe = V * cw1 / G;
  const int64_t v0 = V * cw0 / G + l8;
  if (v0 >= xe) return;
  LtItem cur;
  {
    cur.li = (int)(v0 / ((int64_t)P.h_kv * S));
    const int64_t rem = v0 % ((int64_t)P.h_kv * S);
    cur.h = (int)(rem / S);
    cur.valid = true;
    if (!lt_locate(P, (int)(rem % S), cur)) return;
    lt_fill(P, cur);
  }
  int left = (int)((xe - v0 + Gx - 1) / Gx);

  // Copies row block i of item `it` (its keys, swizzled; its inverse norms)
  // into (Kd, Id): every wavefront 4 KiB of keys, wavefront 0 the norms.
  auto issue = [&](const LtItem& it, int i, char* Kd, float* Id) __attribute__((always_inline)) {
    int ln = threadIdx.x & 63;
    asm volatile("" : "+v"(ln));
    const int page = lt_ld(P.tables, (int64_t)it.r * P.table_stride + i);
    if (page < 0 || page >= P.num_blocks_total) return;  // flagged by phase A
    const int layer = P.layer_begin + it.li;
    const char* kp = reinterpret_cast<const char*>(
        reinterpret_cast<const bf16_t*>(P.kc) + layer * P.kv_layer_elems +
        ((int64_t)page * P.h_kv + it.h) * BT * D);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int pch = (wv * 4 + c4) * 64 + ln;
      const int rr = pch >> 4, c = (pch & 15) ^ (rr & 15);
      __builtin_amdgcn_global_load_lds((lt_gbl_ptr)(kp + rr * L::ROWB + c * 16),
                                       (lt_lds_ptr)(Kd + (wv * 4 + c4) * 1024), 16, 0, 0);
    }
    if (wv == 0) {
      const int64_t zh = (int64_t)(it.li * P.nreq + it.r) * P.h_kv + it.h;
      const float* ip = P.inv + zh * ((int64_t)P.max_blocks * BT) + (int64_t)i * BT;
      __builtin_amdgcn_global_load_lds((lt_gbl_ptr)(ip + ln * 4), (lt_lds_ptr)Id, 16, 0, 0);
    }
  };
  auto item_ok = [&](const LtItem& it) -> bool {
    return it.page >= 0 && it.page < P.num_blocks_total && it.slot >= 0 && it.slot < P.max_slots;
  };

  issue(cur, 0, Ka, Ia);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int buf = 0;  // the buffer that holds the current row block
  for (;;) {
    LtItem nx = cur;
    if (left > 1) lt_skip(P, nx, Gx, layer_count); else nx.valid = false;
    int tid2 = threadIdx.x;
    asm volatile("" : "+v"(tid2));
    const int ln = tid2 & 63, q = ln >> 4, cl = ln & 15;
    const bool ok = item_ok(cur);
    const int z = cur.li * P.nreq + cur.r;
    const int64_t zh = (int64_t)z * P.h_kv + cur.h;
    const int m = cur.pidx, N = cur.N, n = N * BT;
    const int layer = P.layer_begin + cur.li;
    const bf16_t* kbase = reinterpret_cast<const bf16_t*>(P.kc) + layer * P.kv_layer_elems;
    const float* invz = P.inv + zh * ((int64_t)P.max_blocks * BT);
    const float* nrmz = P.nrm + zh * ((int64_t)P.max_blocks * BT);
    const int cg = wv & 7, rh = wv >> 3;
    const int kd = 2 * cg - 8 * rh;  // local row tile of the diagonal tile of c = 0 (block m)
    const bool has_diag = (cg >> 2) == rh;
    // the column block's operands and thresholds, from global memory
    typename M::op_t bop[2][M::NKS];
    float pnc[2], cs[2] = {0.f, 0.f};
    int bk[2] = {-1, -1};  // 32 * row block + 4 * local row tile + v of the highest entry above p
    if (ok) {
      const bf16_t* kpm = kbase + ((int64_t)cur.page * P.h_kv + cur.h) * BT * D;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int col = (2 * cg + c) * 16 + cl;
#pragma unroll
        for (int ks = 0; ks < M::NKS; ++ks) bop[c][ks] = M::glb(kpm + (int64_t)col * D, ks, ln);
        pnc[c] = P.p * nrmz[(int64_t)m * BT + col];
      }
    }
    bool dg[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) dg[v] = 4 * q + v == cl;
    // Row block i from (Kt, It) while the next one is copied into (Kn, In).
    // Called with the two buffers in either order as distinct LDS arrays, so
    // the compiler sees that the copies in flight never alias the reads.
    auto row_block = [&](int i, const char* Kt, const float* It, char* Kn, float* In)
                         __attribute__((always_inline)) {
      if (i + 1 < N) issue(cur, i + 1, Kn, In);
      else if (nx.valid) issue(nx, 0, Kn, In);
      if (ok) {
        const char* Kh = Kt + rh * 128 * L::ROWB;
        const float* ivh = It + rh * 128;
        const bool dblk = i == m;
        const float ivx = wave_max_nq(max_nq(ivh[ln], ivh[ln + 64]));  // over this half's rows
        const float thr[2] = {product_threshold(pnc[0], ivx), product_threshold(pnc[1], ivx)};
        auto load_a = [&](int k, typename M::op_t* a) __attribute__((always_inline)) {
#pragma unroll
          for (int ks = 0; ks < M::NKS; ++ks) a[ks] = M::lds(Kh, k * 16 + cl, ks, ln);
        };
        auto products = [&](const typename M::op_t* a, floatx4* acc) __attribute__((always_inline)) {
          acc[0] = floatx4{0.f, 0.f, 0.f, 0.f};
          acc[1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < M::NKS; ++ks)
#pragma unroll
            for (int c = 0; c < 2; ++c) acc[c] = M::mma(a[ks], bop[c][ks], acc[c]);
        };
        typename M::op_t aA[M::NKS], aB[M::NKS];
        floatx4 accA[2], accB[2];
        float4 ivA, ivB;
        __builtin_amdgcn_s_setprio(3);  // stepped down as the tiles are done (see the lightning kernel)
        load_a(0, aA);
        load_a(1, aB);
        ivA = *reinterpret_cast<const float4*>(ivh + 4 * q);
        products(aA, accA);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (k == 2) __builtin_amdgcn_s_setprio(2);
          if (k == 4) __builtin_amdgcn_s_setprio(1);
          if (k == 6) __builtin_amdgcn_s_setprio(0);
          floatx4* curc = (k & 1) ? accB : accA;
          floatx4* nxt = (k & 1) ? accA : accB;
          typename M::op_t* an = (k & 1) ? aA : aB;
          typename M::op_t* af = (k & 1) ? aB : aA;
          const float4 iv = (k & 1) ? ivB : ivA;
          if (k < 6) load_a(k + 2, af);
          if (k < 7) {
            float4& ivn = (k & 1) ? ivA : ivB;
            ivn = *reinterpret_cast<const float4*>(ivh + (k + 1) * 16 + 4 * q);
            products(an, nxt);
          }
          const float ivv[4] = {iv.x, iv.y, iv.z, iv.w};
          // as in the lightning kernel: the column sums by FMA, the test
          // for an entry above p first against the column's threshold
          float cmx[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            cs[c] = fmaf(curc[c][3], ivv[3], fmaf(curc[c][2], ivv[2], fmaf(curc[c][1], ivv[1], fmaf(curc[c][0], ivv[0], cs[c]))));
            cmx[c] = max_nq(max_nq(curc[c][0], curc[c][1]), max_nq(curc[c][2], curc[c][3]));
          }
          const bool any = !(cmx[0] <= thr[0]) || !(cmx[1] <= thr[1]);
          if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const bool isd = dblk && has_diag && k == kd + c;  // wave-uniform
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const bool hit = curc[c][v] * ivv[v] > pnc[c] && !(isd && dg[v]);
                bk[c] = hit ? 32 * i + 4 * k + v : bk[c];
              }
            }
          }
#pragma unroll
          for (int c = 0; c < 2; ++c) asm volatile("" : "+v"(bk[c]), "+v"(cs[c]));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    for (int i = 0; i < N; ++i) {
      if (buf == 0) row_block(i, Ka, Ia, Kb, Ib);
      else row_block(i, Kb, Ib, Ka, Ia);
      buf ^= 1;
    }
    // per column: over the four row groups, then the two halves of the rows
    if (ok) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int kk = bk[c];
        const int row = kk < 0 ? -1 : (kk >> 5) * BT + (8 * rh + ((kk >> 2) & 7)) * 16 + 4 * q + (kk & 3);
        const int top = xor32_max_i(xor16_max_i(row));
        const int col = (2 * cg + c) * 16 + cl;
        float sum = xor32_sum(xor16_sum(cs[c]));
        // the diagonal entry k_j . k_j / |k_j| = |k_j| out of the sum
        if (has_diag) sum -= nrmz[(int64_t)m * BT + col];
        if (q == 0) {
          crow[rh][col] = top;
          csum[rh][col] = sum;
        }
      }
    }
    __syncthreads();
    if (ok) {  // per column j, four threads of 32 dimensions each
      const int j = tid2 >> 2, part = tid2 & 3;
      const int is = max(crow[0][j], crow[1][j]);
      float d = 0.f;
      if (is >= 0) {
        const int pg = lt_ld(P.tables, (int64_t)cur.r * P.table_stride + is / BT);
        const bf16_t* ki = kbase + ((int64_t)pg * P.h_kv + cur.h) * BT * D + (int64_t)(is % BT) * D;
        const bf16_t* kj = kbase + ((int64_t)cur.page * P.h_kv + cur.h) * BT * D + (int64_t)j * D;
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int c = part * 4; c < part * 4 + 4; ++c) {
          const uint4 u = ld16(ki + c * 8), w = ld16(kj + c * 8);
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.x), __builtin_bit_cast(bf2, w.x), d, false);
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.y), __builtin_bit_cast(bf2, w.y), d, false);
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.z), __builtin_bit_cast(bf2, w.z), d, false);
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.w), __builtin_bit_cast(bf2, w.w), d, false);
        }
      }
      d += dpp_f<DPP_QUAD_XOR1>(d);
      d += dpp_f<DPP_QUAD_XOR2>(d);
      if (part == 0) {
        const float ivj = invz[(int64_t)m * BT + j];
        P.rbuf[zh * ((int64_t)P.max_blocks * BT) + (int64_t)m * BT + j] = (csum[0][j] + csum[1][j]) * ivj;
        if (is >= 0) {
          unsigned long long* rs = P.rsub + zh * ((int64_t)P.max_blocks * BT);
          atomicAdd(rs + is, to_fix(d * invz[is] * ivj));
        }
      }
    }
    __syncthreads();  // csum / crow reused by the next item
    (void)n;
    if (!nx.valid) break;
    cur = nx;
    --left;
  }
}

constexpr size_t kMaxLds = 160 * 1024;  // gfx950 LDS per workgroup

// Compute units of the current device (queried once per device).
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <typename T, int D, int R>
static zp_status launch_score(const ScoreParams& P, int items, hipStream_t s) {
  using L = LdsTile<T, D>;
  const int b = P.b;
  const bool w16 = P.w == 16;
  const bool lse_all = (P.flags & ZP_SCORE_WINDOW_LSE_ALL) != 0;
  const size_t ptileA = ((P.lse_ok || lse_all) && !w16) ? size_t(4) * R * 16 : 0;
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
  bool persistent = false;
  if constexpr (sizeof(T) == 2 && D == 128 && R <= 64) {
    // the serving shape: bf16 keys of head_dim 128 in blocks of 256, a
    // 16-token window, g <= 4 (with flash redundancy: the window scores and
    // the key norms only)
    if (P.b == 256 && P.w == 16) {
      const int64_t work = int64_t(items) * P.h_kv * P.max_blocks;
      const int grid = int(std::min<int64_t>(work, device_cus()));
      hipLaunchKernelGGL(score_lightning_kernel<R / 16>, dim3(grid), dim3(kLtThreads), 0, s, P,
                         items / P.nreq);
      persistent = true;
    }
  }
  if (!persistent) hipLaunchKernelGGL(kA, gridP, dim3(256), smemA, s, P);
  if (flash) {
    bool flash_persistent = false;
    if constexpr (sizeof(T) == 2 && D == 128) {
      if (P.b == 256) {
        const int64_t work = int64_t(items) * P.h_kv * P.max_blocks;
        const int grid = int(std::min<int64_t>(work, device_cus()));
        hipLaunchKernelGGL(score_flash_persist_kernel, dim3(grid), dim3(kLtThreads), 0, s, P,
                           items / P.nreq);
        flash_persistent = true;
      }
    }
    if (!flash_persistent) hipLaunchKernelGGL(kF, gridP, dim3(256), smemF, s, P);
  }
  if (!lse_all) hipLaunchKernelGGL(kB, gridP, dim3(256), smemB, s, P);  // else nothing to gather
  hipLaunchKernelGGL(score_finalize_kernel, dim3(P.h_kv, items), dim3(kFinThreads), 0, s, P);
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
  if ((sp.flags & ZP_SCORE_WINDOW_LSE_ALL) && !cache->qwin_lse)
    return fail(ZP_EINVAL, "zp_score_tokens: ZP_SCORE_WINDOW_LSE_ALL needs cache->qwin_lse");
  if ((sp.flags & ZP_SCORE_GLOBAL) && (!cache->gscore || !f_new))
    return fail(ZP_EINVAL, "zp_score_tokens: ZP_SCORE_GLOBAL needs cache->gscore and f_new");
  if (sp.flags & ~uint32_t(ZP_SCORE_GLOBAL | ZP_SCORE_POOL | ZP_SCORE_POOL_FIRST_ONLY |
                           ZP_SCORE_REDUNDANCY | ZP_SCORE_REDUNDANCY_FLASH | ZP_SCORE_GLOBAL_SUM |
                           ZP_SCORE_WINDOW_LSE_ALL))
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
