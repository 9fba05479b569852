// Per-token importance scores of requests about to be compressed (gfx950).
//
// Zipage (arXiv 2603.08743): App. C.2 Alg. 1 (block attention logits of the
// observation window with a causal mask on the last block; softmax over the
// whole sequence per query head, max over the GQA group, mean over the
// window), App. C.3 Alg. 2 (decayed max-reduce with the global score cache
// F), App. C.4 eq. (3) (max pooling after the global score), App. C.5 eq. (4)
// and C.7 (lightning redundancy: cosine similarity inside each block only,
// diagonal and each column's last entry above p zeroed, row sums over the
// sequence length), App. C.8 (tempered softmax of the redundancy), Sec. 4.2
// (+inf on the observation window).
//
// Three launches per call, all parallel over (block, kv-head, layer x request):
//  A  page_stats: one workgroup per block. The block's keys are staged once
//     in LDS (XOR-swizzled 16-byte chunks, conflict-free MFMA operand reads).
//     MFMA computes the window logits (g*w x b) -> per-row partial (max, sum
//     of exp2) and the block's Gram matrix (b x b) -> lightning row sums.
//  B  page_s0: per block again, merges the row statistics into log-sum-exp,
//     recomputes the logits, forms S0 (group max, window mean) and applies
//     the global score (reads F, writes the updated history to f_new).
//  F  (flash redundancy only) score_flash_redundancy: per column block, Alg. 3
//     over all row blocks, row sums accumulated into the redundancy rows.
//  C  finalize: per (request, kv-head): pooling, redundancy softmax over the
//     sequence, S - lambda R, +inf window -> scores.
// The window QK^T and the Gram are dense contractions (bf16 inputs, fp32
// accumulation on MFMA 16x16x32; fp32 inputs use MFMA 16x16x4 f32).
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

// 16x16 tile C[i][j] = sum_k A[a0 + i][k] * B[b0 + j][k], both operands in LDS.
// Lane l holds C[4*(l/16) + v][l % 16] in element v.
template <typename T, int D>
__device__ floatx4 tile_lds_lds(const char* A, int a0, const char* B, int b0, int lane) {
  using M = Mma<T, D>;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < M::NKS; ++ks)
    acc = M::mma(M::lds(A, a0 + (lane & 15), ks, lane), M::lds(B, b0 + (lane & 15), ks, lane), acc);
  return acc;
}

// Copies `rows` rows of D elements (contiguous in global memory) to an LDS tile.
template <typename T, int D>
__device__ void stage_rows(char* dst, const T* src, int rows, int tid, int nthreads) {
  using L = LdsTile<T, D>;
  const int total = rows * L::CH;
  for (int i = tid; i < total; i += nthreads) {
    const int r = i / L::CH, c = i % L::CH;
    *reinterpret_cast<uint4*>(dst + L::chunk_pos(r, c) * 16) =
        ld16(reinterpret_cast<const char*>(src) + (int64_t)i * 16);
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
  float* scores;
  float* f_new;  // updated global score (S1) per token, same layout as scores
  float* stats;  // [items][h_kv][max_blocks][R][2]  (max, sum) in the exp2 domain
  float* rbuf;   // [items][h_kv][max_blocks * b]     lightning row sums / n
  float* s1buf;  // [items][h_kv][max_blocks * b]     S1
  uint32_t* err;
  int64_t scores_stride;
  int64_t kv_layer_elems, qwin_layer_elems, f_layer_elems;
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

// ---------------------------------------------------------------------------
// Cosine block C = Kr Kc^T of two b x D key blocks staged in LDS (row token i
// of Kr, column token j of Kc): the diagonal is zeroed when `diag` (same
// block), then in every column whose zero-out tag is clear (every column when
// tag == nullptr) the entry of the highest row with C > p is zeroed and the
// tag set, and the rows are summed (Zipage Fig. 11 / Alg. 3 on one pair of
// blocks; the lightning score is the diagonal pair alone). Returns the row
// sum of row `threadIdx.x` (valid for threadIdx.x < b). All 256 threads call
// it; it ends with a barrier, so its LDS scratch may be reused afterwards.
// ---------------------------------------------------------------------------
template <typename T, int D>
__device__ float cosine_block_rows(const char* Kr, const float* inv_r, const char* Kc,
                                   const float* inv_c, bool diag, float p, int* tag, int b,
                                   int* colidx, float* colval, float* rowsum, int* istar,
                                   float* ival) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int q = lane >> 4, cl = lane & 15;
  const int CT = b / 16;
  for (int j = lane; j < b; j += 64) colidx[wv * b + j] = -1;
  for (int rt = wv; rt < CT; rt += 4) {
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};
    for (int ct = 0; ct < CT; ++ct) {
      const floatx4 acc = tile_lds_lds<T, D>(Kr, rt * 16, Kc, ct * 16, lane);
      const int col = ct * 16 + cl;
      const float invc = inv_c[col];
      float c[4];
      uint64_t above[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = rt * 16 + 4 * q + v;
        c[v] = acc[v] * inv_r[row] * invc;
        if (diag && row == col) c[v] = 0.f;
        rsum[v] += c[v];
        above[v] = __ballot(c[v] > p);
      }
      // Highest row of this tile above p in column `col`: row 4*wq + wv2 of
      // the tile, held by the lane of group wq; that lane records it. Rows
      // grow with rt, so a later hit replaces an earlier one.
      int wq = -1, wv2 = 0;
#pragma unroll
      for (int qq = 3; qq >= 0; --qq)
#pragma unroll
        for (int v = 3; v >= 0; --v)
          if (wq < 0 && ((above[v] >> (16 * qq + cl)) & 1ull)) { wq = qq; wv2 = v; }
      if (wq == q) {
        colidx[wv * b + col] = rt * 16 + 4 * wq + wv2;
        colval[wv * b + col] = wv2 == 0 ? c[0] : wv2 == 1 ? c[1] : wv2 == 2 ? c[2] : c[3];
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) rsum[v] = group_sum<16>(rsum[v]);
    if (cl == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) rowsum[rt * 16 + 4 * q + v] = rsum[v];
    }
  }
  __syncthreads();
  if (tid < b) {
    int best = -1;
    float bv = 0.f;
    for (int w2 = 0; w2 < 4; ++w2) {
      const int c = colidx[w2 * b + tid];
      if (c > best) { best = c; bv = colval[w2 * b + tid]; }
    }
    if (tag) {
      if (tag[tid]) best = -1;
      else if (best >= 0) tag[tid] = 1;
    }
    istar[tid] = best;
    ival[tid] = bv;
  }
  __syncthreads();
  float r = 0.f;
  if (tid < b) {
    r = rowsum[tid];
    for (int j = 0; j < b; ++j)
      if (istar[j] == tid) r -= ival[j];
  }
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Phase A: row statistics of the window logits + lightning redundancy rows.
// ---------------------------------------------------------------------------
template <typename T, int D, int R>
__global__ __launch_bounds__(256) void score_page_stats_kernel(ScoreParams P) {
  using L = LdsTile<T, D>;
  constexpr int RT = R / 16;
  extern __shared__ __align__(16) char smem[];
  const int b = P.b;
  char* Ks = smem;                                   // [b][D]
  char* Qs = Ks + b * L::ROWB;                       // [R][D]
  float* inv_norm = reinterpret_cast<float*>(Qs + R * L::ROWB);  // [b]
  float* wstat = inv_norm + b;                       // [4][R][2]
  float* rowsum = wstat + 4 * R * 2;                 // [b]
  int* colidx = reinterpret_cast<int*>(rowsum + b);  // [4][b]
  float* colval = reinterpret_cast<float*>(colidx + 4 * b);  // [4][b]
  int* istar = reinterpret_cast<int*>(colval + 4 * b);       // [b]
  float* ival = reinterpret_cast<float*>(istar + b);         // [b]

  const int pidx = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
  int N, slot;
  const int page = resolve_page(P, pidx, z, &N, &slot);
  if (page < 0) return;
  const int layer = P.layer_begin + z / P.nreq;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool last = pidx == N - 1;
  const int n = N * b;

  const T* kpage = reinterpret_cast<const T*>(P.kc) + layer * P.kv_layer_elems +
                   ((int64_t)page * P.h_kv + h) * b * D;
  const T* qrows = reinterpret_cast<const T*>(P.qwin) + layer * P.qwin_layer_elems +
                   ((int64_t)slot * P.h_kv + h) * R * D;
  stage_rows<T, D>(Ks, kpage, b, tid, 256);
  stage_rows<T, D>(Qs, qrows, R, tid, 256);
  __syncthreads();
  if (tid < b) {
    float ss = 0.f;
    for (int c = 0; c < L::CH; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(Ks + L::chunk_pos(tid, c) * 16);
      float f[Vec16<T>::N];
      Vec16<T>::unpack(v, f);
#pragma unroll
      for (int e = 0; e < Vec16<T>::N; ++e) ss = fmaf(f[e], f[e], ss);
    }
    inv_norm[tid] = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
  }

  // Window logits: this wavefront takes column tiles ct = wv, wv+4, ...
  const int CT = b / 16;
  float rm[RT][4], rs[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) { rm[rt][v] = -INFINITY; rs[rt][v] = 0.f; }
  for (int ct = wv; ct < CT; ct += 4) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const floatx4 acc = tile_lds_lds<T, D>(Qs, rt * 16, Ks, ct * 16, lane);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = rt * 16 + 4 * (lane >> 4) + v;
        const int col = ct * 16 + (lane & 15);
        const int u = row % P.w;
        float x = acc[v] * P.qk_scale;
        if (last && col > b - P.w + u) x = -INFINITY;
        const float tm = group_max<16>(x);
        const float mn = fmaxf(rm[rt][v], tm);
        if (mn != -INFINITY) {
          const float e = group_sum<16>(exp2f(x - mn));
          rs[rt][v] = rs[rt][v] * exp2f(rm[rt][v] - mn) + e;
          rm[rt][v] = mn;
        }
      }
    }
  }
  if ((lane & 15) == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = rt * 16 + 4 * (lane >> 4) + v;
        wstat[(wv * R + row) * 2] = rm[rt][v];
        wstat[(wv * R + row) * 2 + 1] = rs[rt][v];
      }
  }
  __syncthreads();
  const int64_t zh = (int64_t)z * P.h_kv + h;
  if (tid < R) {
    float M = -INFINITY;
    for (int w2 = 0; w2 < 4; ++w2) M = fmaxf(M, wstat[(w2 * R + tid) * 2]);
    float S = 0.f;
    if (M != -INFINITY)
      for (int w2 = 0; w2 < 4; ++w2)
        S += wstat[(w2 * R + tid) * 2 + 1] * exp2f(wstat[(w2 * R + tid) * 2] - M);
    float* st = P.stats + ((zh * P.max_blocks + pidx) * R + tid) * 2;
    st[0] = M;
    st[1] = S;
  }

  if (!(P.flags & ZP_SCORE_REDUNDANCY)) return;
  float* rrow = P.rbuf + zh * ((int64_t)P.max_blocks * b) + (int64_t)pidx * b;
  if (P.flags & ZP_SCORE_REDUNDANCY_FLASH) {
    // Whole-sequence (flash) redundancy: score_flash_redundancy_kernel
    // accumulates into these rows next.
    if (tid < b) rrow[tid] = 0.f;
    return;
  }
  // Lightning redundancy: similarities inside this block only.
  const float r = cosine_block_rows<T, D>(Ks, inv_norm, Ks, inv_norm, true, P.p, nullptr, b,
                                          colidx, colval, rowsum, istar, ival);
  if (tid < b) rrow[tid] = r / (float)n;
}

// ---------------------------------------------------------------------------
// Flash redundancy (Zipage Alg. 3): one workgroup per column block m. Row
// blocks i are visited from the last to the first with one zero-out tag per
// column of m, so each column loses only its highest entry above p over the
// whole sequence; the row sums of every (i, m) pair are added into the row
// sums of block i (the accumulator R'[i][m] summed over m).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void score_flash_redundancy_kernel(ScoreParams P) {
  using L = LdsTile<T, D>;
  extern __shared__ __align__(16) char smem[];
  const int b = P.b;
  char* Km = smem;                                           // [b][D]
  char* Ki = Km + b * L::ROWB;                               // [b][D]
  float* inv_m = reinterpret_cast<float*>(Ki + b * L::ROWB); // [b]
  float* inv_i = inv_m + b;                                  // [b]
  int* tag = reinterpret_cast<int*>(inv_i + b);              // [b]
  int* colidx = tag + b;                                     // [4][b]
  float* colval = reinterpret_cast<float*>(colidx + 4 * b);  // [4][b]
  float* rowsum = colval + 4 * b;                            // [b]
  int* istar = reinterpret_cast<int*>(rowsum + b);           // [b]
  float* ival = reinterpret_cast<float*>(istar + b);         // [b]

  const int m = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
  int N, slot;
  const int page_m = resolve_page(P, m, z, &N, &slot);
  if (page_m < 0) return;
  const int r = z % P.nreq;
  const int layer = P.layer_begin + z / P.nreq;
  const int tid = threadIdx.x;
  const int n = N * b;
  const int64_t zh = (int64_t)z * P.h_kv + h;
  const T* kbase = reinterpret_cast<const T*>(P.kc) + layer * P.kv_layer_elems;
  const int32_t* tab = P.tables + (int64_t)r * P.table_stride;
  for (int i = 0; i < N; ++i) {          // all block ids were checked by phase A
    const int pg = tab[i];
    if (pg < 0 || pg >= P.num_blocks_total) return;
  }
  auto stage = [&](char* dst, float* inv, int page) {
    stage_rows<T, D>(dst, kbase + ((int64_t)page * P.h_kv + h) * b * D, b, tid, 256);
    __syncthreads();
    if (tid < b) {
      float ss = 0.f;
      for (int c = 0; c < L::CH; ++c) {
        const uint4 v = *reinterpret_cast<const uint4*>(dst + L::chunk_pos(tid, c) * 16);
        float f[Vec16<T>::N];
        Vec16<T>::unpack(v, f);
#pragma unroll
        for (int e = 0; e < Vec16<T>::N; ++e) ss = fmaf(f[e], f[e], ss);
      }
      inv[tid] = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
    }
  };
  stage(Km, inv_m, page_m);
  if (tid < b) tag[tid] = 0;
  __syncthreads();
  float* rb = P.rbuf + zh * ((int64_t)P.max_blocks * b);
  for (int i = N - 1; i >= 0; --i) {
    const bool same = i == m;
    if (!same) {
      stage(Ki, inv_i, tab[i]);
      __syncthreads();
    }
    const float rs = cosine_block_rows<T, D>(same ? Km : Ki, same ? inv_m : inv_i, Km, inv_m, same,
                                             P.p, tag, b, colidx, colval, rowsum, istar, ival);
    if (tid < b) atomicAdd(rb + (int64_t)i * b + tid, rs / (float)n);
  }
}

// ---------------------------------------------------------------------------
// Phase B: S0 of one block (App. C.2) and the global score (Alg. 2).
// ---------------------------------------------------------------------------
template <typename T, int D, int R>
__global__ __launch_bounds__(256) void score_page_s0_kernel(ScoreParams P) {
  using L = LdsTile<T, D>;
  using M = Mma<T, D>;
  constexpr int RT = R / 16;
  extern __shared__ __align__(16) char smem[];
  char* Qs = smem;                                           // [R][D]
  float* lse2 = reinterpret_cast<float*>(Qs + R * L::ROWB);  // [R]
  float* ptile = lse2 + R;                                   // [4][R][16]

  const int pidx = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
  int N, slot;
  const int page = resolve_page(P, pidx, z, &N, &slot);
  if (page < 0) return;
  const int r = z % P.nreq;
  const int layer = P.layer_begin + z / P.nreq;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = P.b;
  const bool last = pidx == N - 1;
  const int64_t zh = (int64_t)z * P.h_kv + h;

  const T* qrows = reinterpret_cast<const T*>(P.qwin) + layer * P.qwin_layer_elems +
                   ((int64_t)slot * P.h_kv + h) * R * D;
  stage_rows<T, D>(Qs, qrows, R, tid, 256);
  if (tid < R) {
    const float* st = P.stats + (zh * P.max_blocks) * R * 2 + tid * 2;
    float Mx = -INFINITY;
    for (int q = 0; q < N; ++q) Mx = fmaxf(Mx, st[(int64_t)q * R * 2]);
    float S = 0.f;
    for (int q = 0; q < N; ++q) S += st[(int64_t)q * R * 2 + 1] * exp2f(st[(int64_t)q * R * 2] - Mx);
    lse2[tid] = Mx + log2f(S);
  }
  __syncthreads();

  const T* kpage = reinterpret_cast<const T*>(P.kc) + layer * P.kv_layer_elems +
                   ((int64_t)page * P.h_kv + h) * b * D;
  const int G = R / P.w;
  const bool first = P.first[r] != 0;
  float* ptw = ptile + wv * R * 16;
  for (int ct = wv; ct < b / 16; ct += 4) {
    const T* krow = kpage + (int64_t)(ct * 16 + (lane & 15)) * D;
    typename M::op_t bop[M::NKS];
#pragma unroll
    for (int ks = 0; ks < M::NKS; ++ks) bop[ks] = M::glb(krow, ks, lane);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < M::NKS; ++ks)
        acc = M::mma(M::lds(Qs, rt * 16 + (lane & 15), ks, lane), bop[ks], acc);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = rt * 16 + 4 * (lane >> 4) + v;
        const int col = ct * 16 + (lane & 15);
        const int u = row % P.w;
        float pv = exp2f(acc[v] * P.qk_scale - lse2[row]);
        if (last && col > b - P.w + u) pv = 0.f;
        ptw[row * 16 + (lane & 15)] = pv;
      }
    }
    // Within a wavefront LDS writes and reads are ordered; no barrier needed.
    if (lane < 16) {
      const int col = ct * 16 + lane;
      float s0 = 0.f;
      for (int u = 0; u < P.w; ++u) {
        float mx = 0.f;
        for (int gi = 0; gi < G; ++gi) mx = fmaxf(mx, ptw[(gi * P.w + u) * 16 + lane]);
        s0 += mx;
      }
      s0 /= (float)P.w;
      float s1 = s0;
      if (P.flags & ZP_SCORE_GLOBAL) {
        // F is read only: blocks may be shared by several requests.
        if (!first && !last)
          s1 = fmaxf(P.alpha * P.gscore[layer * P.f_layer_elems + ((int64_t)page * P.h_kv + h) * b + col], s0);
        P.f_new[zh * P.scores_stride + (int64_t)pidx * b + col] = s1;
      }
      P.s1buf[zh * ((int64_t)P.max_blocks * b) + (int64_t)pidx * b + col] = s1;
    }
  }
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
  const float* rr = P.rbuf + zh * ((int64_t)P.max_blocks * P.b);
  float* out = P.scores + zh * P.scores_stride;
  const bool first = P.first[r] != 0;
  const bool pool = (P.flags & ZP_SCORE_POOL) && (first || !(P.flags & ZP_SCORE_POOL_FIRST_ONLY));
  const bool redun = (P.flags & ZP_SCORE_REDUNDANCY) != 0;
  const int half = P.pool_kernel / 2;
  const float c2 = P.inv_tau * kLog2e;  // softmax(r / tau) in the exp2 domain

  float mx = -INFINITY, sum = 0.f;
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
  const size_t smemA = size_t(b) * L::ROWB + size_t(R) * L::ROWB +
                       sizeof(float) * (b + 4 * R * 2 + b) + sizeof(int) * 4 * b +
                       sizeof(float) * 4 * b + sizeof(int) * b + sizeof(float) * b;
  const size_t smemB = size_t(R) * L::ROWB + sizeof(float) * (R + 4 * R * 16);
  if (smemA > kMaxLds || smemB > kMaxLds)
    return fail(ZP_EINVAL, "zp_score_tokens: block_size %d with this dtype/head_dim needs %zu "
                "bytes of LDS (max %zu)", b, smemA, kMaxLds);
  const bool flash = (P.flags & ZP_SCORE_REDUNDANCY) && (P.flags & ZP_SCORE_REDUNDANCY_FLASH);
  const size_t smemF = 2 * size_t(b) * L::ROWB + sizeof(float) * 2 * b + sizeof(int) * b +
                       sizeof(int) * 4 * b + sizeof(float) * 4 * b + sizeof(float) * b +
                       sizeof(int) * b + sizeof(float) * b;
  if (flash && smemF > kMaxLds)
    return fail(ZP_EINVAL, "zp_score_tokens: flash redundancy with block_size %d and this "
                "dtype/head_dim needs %zu bytes of LDS (max %zu)", b, smemF, kMaxLds);
  auto kA = score_page_stats_kernel<T, D, R>;
  auto kB = score_page_s0_kernel<T, D, R>;
  auto kF = score_flash_redundancy_kernel<T, D>;
  if (flash && hipFuncSetAttribute(reinterpret_cast<const void*>(kF),
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   int(smemF)) != hipSuccess)
    return fail(ZP_EHIP, "zp_score_tokens: cannot reserve %zu bytes of LDS", smemF);
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kA),
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(smemA)) != hipSuccess ||
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
                              size_t* s1_off) {
  const size_t items = size_t(layer_count) * nreq * g->num_kv_heads;
  const size_t R = size_t(group_size(g)) * g->window;
  const size_t per_tok = size_t(max_blocks) * g->block_size;
  const size_t st = kWsHeader;
  const size_t ro = round_up(st + items * max_blocks * R * 2 * sizeof(float), 256);
  const size_t so = round_up(ro + items * per_tok * sizeof(float), 256);
  const size_t total = round_up(so + items * per_tok * sizeof(float), 256);
  if (stats_off) *stats_off = st;
  if (r_off) *r_off = ro;
  if (s1_off) *s1_off = so;
  return total;
}

}  // namespace zp

using namespace zp;

extern "C" size_t zp_score_workspace_size(const zp_geom* geom, int32_t layer_count, int32_t nreq,
                                          int32_t max_blocks) {
  if (validate_geom(geom, "zp_score_workspace_size") != ZP_OK || layer_count < 0 || nreq < 0 ||
      max_blocks < 0)
    return 0;
  return score_ws_layout(geom, layer_count, nreq, max_blocks, nullptr, nullptr, nullptr);
}

extern "C" zp_status zp_score_tokens(const zp_geom* geom, const zp_cache* cache,
                                     const zp_score_params* params, int32_t layer_begin,
                                     int32_t layer_count, int32_t nreq,
                                     const int32_t* block_tables, int32_t table_stride,
                                     const int32_t* num_blocks, int32_t max_blocks,
                                     const int32_t* qslot, const uint8_t* first_compression,
                                     float* scores, float* f_new, int64_t scores_stride,
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
  if ((sp.flags & ZP_SCORE_GLOBAL) && (!cache->gscore || !f_new))
    return fail(ZP_EINVAL, "zp_score_tokens: ZP_SCORE_GLOBAL needs cache->gscore and f_new");
  if (sp.flags & ~uint32_t(ZP_SCORE_GLOBAL | ZP_SCORE_POOL | ZP_SCORE_POOL_FIRST_ONLY |
                           ZP_SCORE_REDUNDANCY | ZP_SCORE_REDUNDANCY_FLASH))
    return fail(ZP_EINVAL, "zp_score_tokens: unknown flags 0x%x", sp.flags);
  if ((sp.flags & ZP_SCORE_POOL) && (sp.pool_kernel < 1 || sp.pool_kernel % 2 == 0))
    return fail(ZP_EINVAL, "zp_score_tokens: pool_kernel must be odd and >= 1");
  if ((sp.flags & ZP_SCORE_REDUNDANCY) && !(sp.tau > 0.f))
    return fail(ZP_EINVAL, "zp_score_tokens: tau must be > 0");
  if ((sp.flags & ZP_SCORE_REDUNDANCY) && !(sp.sim_threshold >= 0.f))
    return fail(ZP_EINVAL, "zp_score_tokens: sim_threshold must be >= 0");
  if (geom->max_slots <= 0) return fail(ZP_EINVAL, "zp_score_tokens: no query slots");
  size_t so, ro, s1o;
  const size_t need = score_ws_layout(geom, layer_count, nreq, max_blocks, &so, &ro, &s1o);
  if (workspace_bytes < need)
    return fail(ZP_EINVAL, "zp_score_tokens: workspace %zu bytes, need %zu", workspace_bytes, need);
  const int64_t items = int64_t(layer_count) * nreq;
  if (items > 65535) return fail(ZP_EINVAL, "zp_score_tokens: layer_count*nreq > 65535");

  ScoreParams P{};
  P.kc = cache->k; P.qwin = cache->qwin; P.gscore = cache->gscore;
  P.tables = block_tables; P.num_blocks = num_blocks; P.qslot = qslot;
  P.first = first_compression; P.scores = scores; P.f_new = f_new;
  P.scores_stride = scores_stride;
  char* ws = static_cast<char*>(workspace);
  P.err = reinterpret_cast<uint32_t*>(ws);
  P.stats = reinterpret_cast<float*>(ws + so);
  P.rbuf = reinterpret_cast<float*>(ws + ro);
  P.s1buf = reinterpret_cast<float*>(ws + s1o);
  const int64_t d = geom->head_dim;
  P.kv_layer_elems = int64_t(geom->num_blocks) * geom->num_kv_heads * geom->block_size * d;
  P.qwin_layer_elems = int64_t(geom->max_slots) * geom->num_q_heads * geom->window * d;
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
