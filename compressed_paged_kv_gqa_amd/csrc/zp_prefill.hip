// Paged causal prefill attention for gfx950 (one layer, a ragged batch of
// prompt chunks).
//
// Zipage (arXiv 2603.08743): Sec. 3 (K/V in fixed-size blocks addressed
// through per-request block tables), Sec. 4.1 (a prompt is written in full
// and may exceed the N_max-block cap until its first compression), Sec. 4.2
// (the queries of the last w slots of the final block are kept in the query
// cache), Sec. 4.4 (a request may start from shared prefix blocks, so a chunk
// attends to ctx tokens already resident), Sec. 6 (eviction leaves attention
// as ordinary causal softmax attention).
//
// Two launches:
//  1. prefill_append_kernel: the chunk's K/V rows go to their blocks; the
//     window queries of the final block go to the query cache.
//  2. Attention. bf16: prefill_attn_kernel, one workgroup per (tile of
//     128/g query tokens, kv-head, request), all g query heads of the kv-head
//     in one workgroup so every K/V tile read serves 128 query rows. Per tile
//     of 64 keys (prefetched into registers while the previous tile is being
//     used) MFMA forms S^T = K Q^T, so each lane holds the logits of one
//     query and the online softmax needs only two cross-group shuffles; then
//     O^T += V^T P^T, with V staged transposed in LDS and P taken straight
//     from the registers that hold it (the k-ordering of the product follows
//     P's register layout). fp32: prefill_simple_kernel, one workgroup per
//     (token, kv-head, request), a decode-style pass over the causal prefix.
//     Both emit the log-sum-exp of every row; window rows of the final block
//     also go to the query cache's LSE table.
#include <cmath>

#include "zp_device.h"
#include "zp_internal.h"

namespace zp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct PrefillParams {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* kc;
  void* vc;
  void* qwin;
  float* qwin_lse;
  const int32_t* cu;
  const int32_t* ctx;
  const int32_t* tables;
  const int32_t* qslot;
  void* out;
  float* lse;
  uint32_t* err;
  int64_t kv_layer_off;    // element offset of the layer in K / V
  int64_t qwin_layer_off;  // element offset of the layer in the query cache
  int64_t qlse_layer_off;  // element offset of the layer in the query-cache LSE table
  int32_t nreq, table_stride, num_blocks, b, h_kv, w, max_slots, max_q_len, log2b;
  float qk_scale;  // log2(e) / sqrt(d)
};

// Chunk geometry of request r; false (and an error bit, set by the
// workgroups with `lead`) when it does not fit.
__device__ __forceinline__ bool chunk_of(const PrefillParams& P, int r, int* c0, int* qlen,
                                         int* ctx, bool lead) {
  const int a = P.cu[r], e = P.cu[r + 1], cx = P.ctx[r];
  if (e < a || e - a > P.max_q_len || cx < 0 ||
      (int64_t)cx + (e - a) > (int64_t)P.table_stride * P.b) {
    if (threadIdx.x == 0 && lead) flag_error(P.err, ZP_DEVERR_SEQ_LEN);
    return false;
  }
  *c0 = a;
  *qlen = e - a;
  *ctx = cx;
  return true;
}

// Window row of position pos in the final block of a chunk that ends at
// position last (inclusive), or -1.
__device__ __forceinline__ int window_row(const PrefillParams& P, int pos, int last) {
  const int b = P.b;
  if ((pos >> P.log2b) != (last >> P.log2b)) return -1;
  const int off = pos & (b - 1);
  return off >= b - P.w ? off - (b - P.w) : -1;
}

// ---------------------------------------------------------------------------
// 1. Append the chunk's K/V; capture the final block's window queries.
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void prefill_append_kernel(PrefillParams P) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPR = D / EPL;    // lanes per row
  constexpr int RPP = 256 / LPR;  // rows per pass
  const int r = blockIdx.z, h = blockIdx.y, i0 = blockIdx.x * 64;
  int c0, qlen, ctx;
  if (!chunk_of(P, r, &c0, &qlen, &ctx, blockIdx.x == 0) || i0 >= qlen) return;
  const int tid = threadIdx.x, sub = tid % LPR;
  const int32_t* tab = P.tables + (int64_t)r * P.table_stride;
  const int last = ctx + qlen - 1;
  int slot = -1;
  if (P.qslot) {
    slot = P.qslot[r];  // negative: no query slot, nothing captured
    if (slot >= P.max_slots) {
      if (tid == 0) flag_error(P.err, ZP_DEVERR_SLOT);
      slot = -1;
    }
  }
  T* kc = reinterpret_cast<T*>(P.kc) + P.kv_layer_off;
  T* vc = reinterpret_cast<T*>(P.vc) + P.kv_layer_off;
  const T* kn = reinterpret_cast<const T*>(P.k_new);
  const T* vn = reinterpret_cast<const T*>(P.v_new);
  for (int row = tid / LPR; row < 64; row += RPP) {
    const int i = i0 + row;
    if (i >= qlen) break;
    const int pos = ctx + i;
    const int page = tab[pos >> P.log2b];
    if (page < 0 || page >= P.num_blocks) {
      if (sub == 0) flag_error(P.err, ZP_DEVERR_BLOCK_ID);
      continue;
    }
    const int64_t dst = (((int64_t)page * P.h_kv + h) * P.b + (pos & (P.b - 1))) * D + sub * EPL;
    const int64_t src = ((int64_t)(c0 + i) * P.h_kv + h) * D + sub * EPL;
    st16(kc + dst, ld16(kn + src));
    st16(vc + dst, ld16(vn + src));
    const int u = slot >= 0 ? window_row(P, pos, last) : -1;
    if (u >= 0) {
      const T* qs = reinterpret_cast<const T*>(P.q) + ((int64_t)(c0 + i) * P.h_kv * G + h * G) * D;
      T* qd = reinterpret_cast<T*>(P.qwin) + P.qwin_layer_off +
              (((int64_t)slot * P.h_kv + h) * G) * P.w * D + (int64_t)u * D;
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
        st16(qd + (int64_t)gi * P.w * D + sub * EPL, ld16(qs + gi * D + sub * EPL));
    }
  }
}

// Writes the log-sum-exp of (token i, head gi) of request r: to lse[] and,
// for window rows of the final block, to the query-cache LSE table.
__device__ __forceinline__ void emit_lse(const PrefillParams& P, int r, int c0, int i, int pos,
                                         int last, int h, int G, int gi, float lse_nat) {
  const int hq = h * G + gi;
  if (P.lse) P.lse[(int64_t)(c0 + i) * P.h_kv * G + hq] = lse_nat;
  if (P.qslot && P.qwin_lse) {
    const int slot = P.qslot[r];
    const int u = window_row(P, pos, last);
    if (u >= 0 && slot >= 0 && slot < P.max_slots)
      P.qwin_lse[P.qlse_layer_off + (((int64_t)slot * P.h_kv + h) * G + gi) * P.w + u] = lse_nat;
  }
}

// ---------------------------------------------------------------------------
// 2a. bf16 attention on MFMA.
// ---------------------------------------------------------------------------
constexpr int kPKT = 64;                 // keys per tile
constexpr float kPLazy = 8.0f;           // lazy rescale threshold (log2 units)
// The bf16 kernels form a tile's weights with the running maximum as it
// stands and move the maximum only when a lane's partial sum of its n
// weights exceeds n * 2^kPLazy, i.e. at latest when some weight would pass
// 2^kPLazy; every weight stays below n * 2^kPLazy (2^11 with 32-key tiles,
// 2^12 with 64), which fp32 sums and bf16 weights hold.
constexpr float psum_cap(int weights_per_lane) { return 256.0f * weights_per_lane; }  // 2^kPLazy
static_assert(kPLazy == 8.0f, "psum_cap assumes 2^kPLazy = 256");
constexpr int kPRows = 128;              // query rows (token, head) per workgroup
constexpr int kPfTabLds = 2048;          // block ids staged in LDS (tables up to this wide)
#ifndef ZP_PF_DMA_KT
#define ZP_PF_DMA_KT 32
#endif
constexpr int kPfDmaKT = ZP_PF_DMA_KT;   // keys per tile of the LDS-copy kernel
constexpr int kVtStride = kPKT + 4;      // bf16 per row of the transposed V tile
// Key slot of key `key` in row d of the transposed V tile: XOR with a
// multiple of 4 keyed by d / 8, so the dword writes of lanes that hold
// different 8-dim chunks fall in distinct banks while every group of 4
// consecutive keys stays contiguous for the 8-byte operand reads.
__device__ __forceinline__ int vt_slot(int d, int key) { return key ^ (((d >> 3) & 15) << 2); }

template <int D>
struct PfTile {
  static constexpr int CH = D * 2 / 16;  // 16-byte chunks per key row
  static constexpr int SW = CH < 16 ? CH : 16;
  static constexpr int ROWB = CH * 16;
  __device__ static int chunk_pos(int r, int c) { return r * CH + (c ^ (r % SW)); }
  // loads per thread for one tile of K (and of V): pairs of key rows
  static constexpr int PAIRS = kPKT / 2 * CH / 256;
};

template <int D, int G>
__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(PrefillParams P) {
  using L = PfTile<D>;
  constexpr int QT = kPRows / G;   // query tokens per workgroup
  constexpr int NDT = D / 16;      // output column tiles (head dims)
  constexpr int NKS = D / 32;      // k-steps of the logits
  __shared__ __align__(16) char Ks[kPKT * L::ROWB];
  __shared__ __align__(16) bf16_t Vt[D * kVtStride];

  const int r = blockIdx.z, h = blockIdx.y;
  int c0, qlen, ctx;
  if (!chunk_of(P, r, &c0, &qlen, &ctx, blockIdx.x == 0)) return;
  const int ntq = (P.max_q_len + QT - 1) / QT;
  const int qt = ntq - 1 - blockIdx.x;            // heavy (late) tiles first
  const int q0 = qt * QT;
  if (q0 >= qlen) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, cl = lane & 15;
  const int q_last = min(qlen, q0 + QT) - 1;
  const int n_keys = ctx + q_last + 1;             // keys any row of the tile may see
  const int ntiles = (n_keys + kPKT - 1) / kPKT;
  const int32_t* tab = P.tables + (int64_t)r * P.table_stride;
  const bf16_t* kcache = reinterpret_cast<const bf16_t*>(P.kc) + P.kv_layer_off;
  const bf16_t* vcache = reinterpret_cast<const bf16_t*>(P.vc) + P.kv_layer_off;
  const int h_q = P.h_kv * G;

  // This wavefront's two row tiles: rows rt * 16 + j = (head gi, token ti).
  int gi_of[2], ti0_of[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int row0 = (2 * wv + k) * 16;
    gi_of[k] = row0 / QT;
    ti0_of[k] = row0 % QT;
  }
  // Q operands (B of S^T = K Q^T): lane holds query ti0 + cl, k-slice q.
  bf16x8_t qop[2][NKS];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = min(q0 + ti0_of[k] + cl, qlen - 1);  // rows past the chunk are discarded
    const bf16_t* qr = reinterpret_cast<const bf16_t*>(P.q) +
                       ((int64_t)(c0 + i) * h_q + h * G + gi_of[k]) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qop[k][ks] = __builtin_bit_cast(bf16x8_t, ld16(qr + ks * 32 + q * 8));
  }

  // K/V tile staging: thread -> (key pair kp, 16-byte chunk cc). The block
  // ids of a tile are looked up one tile ahead of its K/V loads, and every
  // load is issued unconditionally (keys past n_keys or on a bad block read
  // a row that exists and are zeroed when staged), so no wait on the lookups
  // or on an earlier tile stalls the loads in flight.
  uint4 kr[L::PAIRS][2], vr[L::PAIRS][2];
  int pg[L::PAIRS][2];
  uint32_t live = 0;  // bit 2j+e: key (j, e) of the loaded tile is resident
  bool bad = false;   // a needed key sits on an out-of-range block id
  auto lookup = [&](int t) {
#pragma unroll
    for (int j = 0; j < L::PAIRS; ++j) {
      const int kp = (tid + 256 * j) / L::CH;
#pragma unroll
      for (int e = 0; e < 2; ++e) pg[j][e] = tab[min(t * kPKT + 2 * kp + e, n_keys - 1) >> P.log2b];
    }
  };
  auto load_tile = [&](int t) {
    live = 0;
#pragma unroll
    for (int j = 0; j < L::PAIRS; ++j) {
      const int idx = tid + 256 * j;
      const int kp = idx / L::CH, cc = idx % L::CH;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int pos = t * kPKT + 2 * kp + e, page = pg[j][e];
        const bool ok = page >= 0 && page < P.num_blocks;
        bad |= pos < n_keys && !ok;
        const bool use = pos < n_keys && ok;
        live |= uint32_t(use) << (2 * j + e);
        // cache row (block, head, slot): fits 32 bits, as a layer's rows
        // times 2D bytes is far below 2^31 * 256 bytes
        const uint32_t row = use ? ((uint32_t)page * P.h_kv + h) * P.b + (pos & (P.b - 1)) : 0u;
        const int64_t off = (int64_t)row * D + cc * 8;
        kr[j][e] = ld16(kcache + off);
        vr[j][e] = ld16(vcache + off);
      }
    }
  };
  auto store_tile = [&]() {
    if (live != (1u << (2 * L::PAIRS)) - 1u) {  // tail tile or bad block: stage zeros
#pragma unroll
      for (int j = 0; j < L::PAIRS; ++j)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          if (!((live >> (2 * j + e)) & 1u)) {
            kr[j][e].x = kr[j][e].y = kr[j][e].z = kr[j][e].w = 0u;
            vr[j][e].x = vr[j][e].y = vr[j][e].z = vr[j][e].w = 0u;
          }
    }
#pragma unroll
    for (int j = 0; j < L::PAIRS; ++j) {
      const int idx = tid + 256 * j;
      const int kp = idx / L::CH, cc = idx % L::CH;
#pragma unroll
      for (int e = 0; e < 2; ++e)
        *reinterpret_cast<uint4*>(Ks + L::chunk_pos(2 * kp + e, cc) * 16) = kr[j][e];
      // V transposed: Vt[d][key], keys 2kp and 2kp+1 packed in one dword
      const uint32_t a[4] = {vr[j][0].x, vr[j][0].y, vr[j][0].z, vr[j][0].w};
      const uint32_t c[4] = {vr[j][1].x, vr[j][1].y, vr[j][1].z, vr[j][1].w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int d = cc * 8 + 2 * x;  // d and d + 1 share d / 8
        const int ks = vt_slot(d, 2 * kp);
        *reinterpret_cast<uint32_t*>(&Vt[d * kVtStride + ks]) = __builtin_amdgcn_perm(c[x], a[x], 0x05040100u);
        *reinterpret_cast<uint32_t*>(&Vt[(d + 1) * kVtStride + ks]) = __builtin_amdgcn_perm(c[x], a[x], 0x07060302u);
      }
    }
  };

  floatx4 o[2][NDT];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[k][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-1.0e30f, -1.0e30f}, l[2] = {0.f, 0.f};
  int qpos[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) qpos[k] = ctx + q0 + ti0_of[k] + cl;  // this lane's query position

  lookup(0);
  load_tile(0);
  lookup(min(1, ntiles - 1));
  store_tile();
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) load_tile(t + 1);  // in flight while this tile is used
    lookup(min(t + 2, ntiles - 1));
    const bool diag = t * kPKT + kPKT - 1 > ctx + q0;  // some key may follow some query
    bf16x8_t pop[2][2];
    // Logits of both row tiles: each K operand read from LDS feeds two MFMAs.
    floatx4 sk[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) sk[k][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int c = ks * 4 + q;
        const bf16x8_t kop = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(Ks + L::chunk_pos(ct * 16 + cl, c) * 16));
        sk[0][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[0][ks], sk[0][ct], 0, 0, 0);
        sk[1][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[1][ks], sk[1][ct], 0, 0, 0);
      }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      floatx4 (&s)[4] = sk[k];
      // s[ct][v] = raw logit of key t*64 + ct*16 + 4q + v for this lane's
      // query; softmax in the exp2 domain with the scale folded into an FMA.
      // m is the running max of the scaled logits, raised (and O, l
      // rescaled) only when a weight exp2(x - m) would grow too large.
      if (diag) {  // one branch, taken on the last tile or two only
        const int lim = qpos[k] - t * kPKT - 4 * q;  // last visible key offset
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (ct * 16 + v > lim) s[ct][v] = -INFINITY;
      }
      // weights against the running maximum as it stands; the tile's row
      // maxima only when a weight would pass 2^kPLazy (see psum_cap)
      float ps = 0.f;
      float p[4][4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          p[ct][v] = __builtin_amdgcn_exp2f(fmaf(s[ct][v], P.qk_scale, -m[k]));
          ps += p[ct][v];
        }
      if (__builtin_amdgcn_read_exec() & __ballot(!(ps <= psum_cap(16)))) {
        float mx = -INFINITY;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[ct][v]);
        mx = xor32_max(xor16_max(mx));
        mx *= P.qk_scale;
        const float mn = fmaxf(m[k], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[k] - mn);
        m[k] = mn;
        l[k] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[k][dt] *= alpha;
        ps = 0.f;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            p[ct][v] = __builtin_amdgcn_exp2f(fmaf(s[ct][v], P.qk_scale, -m[k]));
            ps += p[ct][v];
          }
      }
      l[k] += ps;
      // P operands: k-step st holds keys {32st + 4q + v} and {32st + 16 + 4q + v}
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        b2 x0 = __builtin_convertvector(f2{p[2 * st][0], p[2 * st][1]}, b2);
        b2 x1 = __builtin_convertvector(f2{p[2 * st][2], p[2 * st][3]}, b2);
        b2 x2 = __builtin_convertvector(f2{p[2 * st + 1][0], p[2 * st + 1][1]}, b2);
        b2 x3 = __builtin_convertvector(f2{p[2 * st + 1][2], p[2 * st + 1][3]}, b2);
        const uint4 u = make_uint4(__builtin_bit_cast(uint32_t, x0), __builtin_bit_cast(uint32_t, x1),
                                   __builtin_bit_cast(uint32_t, x2), __builtin_bit_cast(uint32_t, x3));
        pop[k][st] = __builtin_bit_cast(bf16x8_t, u);
      }
    }
    // O^T += V^T P^T: A = V^T rows d = dt*16 + cl, same key order as P.
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d = dt * 16 + cl;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint2 lo = *reinterpret_cast<const uint2*>(&Vt[d * kVtStride + vt_slot(d, 32 * st + 4 * q)]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&Vt[d * kVtStride + vt_slot(d, 32 * st + 16 + 4 * q)]);
        const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int k = 0; k < 2; ++k)
          o[k][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[k][st], o[k][dt], 0, 0, 0);
      }
    }
    __syncthreads();  // every wavefront is done with this tile
    if (t + 1 < ntiles) {
      store_tile();
      __syncthreads();
    }
  }

  if (bad) flag_error(P.err, ZP_DEVERR_BLOCK_ID);
  // Finish: the four lane groups hold partial sums of each query's weights.
  const int last = ctx + qlen - 1;
  bf16_t* out = reinterpret_cast<bf16_t*>(P.out);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float lt = xor32_sum(xor16_sum(l[k]));
    const int i = q0 + ti0_of[k] + cl;
    if (i >= qlen) continue;
    const float inv = 1.0f / lt;
    bf16_t* orow = out + ((int64_t)(c0 + i) * h_q + h * G + gi_of[k]) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      // o[k][dt][v] = O[query][dt*16 + 4q + v]
      const uint32_t w0 = uint32_t(f32_to_bf16(o[k][dt][0] * inv)) | (uint32_t(f32_to_bf16(o[k][dt][1] * inv)) << 16);
      const uint32_t w1 = uint32_t(f32_to_bf16(o[k][dt][2] * inv)) | (uint32_t(f32_to_bf16(o[k][dt][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(orow + dt * 16 + 4 * q) = make_uint2(w0, w1);
    }
    if (q == 0) emit_lse(P, r, c0, i, ctx + i, last, h, G, gi_of[k], (m[k] + log2f(lt)) * kLn2);
  }
}

// ---------------------------------------------------------------------------
// 2a'. bf16 attention with K/V tiles copied straight into LDS (blocks of at
// least KT tokens, block table staged in LDS).
//
// The loads of a tile go from HBM to LDS without registers
// (global_load_lds, 16 bytes per lane): K in 16-byte chunks XOR-swizzled
// like the register path; V with each row's 32-byte segments permuted by
// the row index (vseg), the lanes of one copy fetching whichever chunk its
// destination slot holds. The V^T operand of the PV product is then read
// with the transposing LDS load (ds_read_b64_tr_b16): within each group of
// 16 lanes, lane l receives element l % 4 of the 8-byte pieces addressed by
// lanes l / 4, l / 4 + 4, l / 4 + 8, l / 4 + 12. Lane (cl, q) addresses row
// 4q + cl / 4 (plus the tile's key offset), columns d = 16dt + 4(cl % 4) ..
// +3, and so receives V[4 consecutive keys][16dt + cl]: the A operand of O^T
// += V^T P^T in the key order of the P registers. The 16 rows one read
// touches fall evenly on the four 128-byte bank windows.
//
// Two LDS buffers alternate: tile t + 1 is in flight while tile t is used,
// and one barrier per tile both retires the copies (the barrier waits for
// them) and frees the buffer the next copy overwrites.
//
// Key tiles of 32 (KT): a workgroup then needs 40 KB of LDS and 168 VGPRs
// per lane, so three workgroups share a CU (three wavefronts per SIMD). On
// this kernel MFMA and VALU time add up on a SIMD, and the third wavefront
// hides more of the LDS and copy latency than the extra per-tile work of the
// shorter tile costs (64-key tiles fit two workgroups per CU).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* gbl_void_ptr;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t* lds_v4i16_ptr;

template <int D, int KT>
struct PfDma {
  static constexpr int CH = D * 2 / 16;          // 16-byte chunks per key row
  static constexpr int KB = KT * D * 2;          // bytes of a K (or V) tile
  static constexpr int KI = KB / 1024 / 4;       // 1 KiB copies per wavefront per tile
  static constexpr int VS = D * 2;               // bytes per V row
  static constexpr int NSEG = D * 2 / 32;        // 32-byte segments per V row
  __device__ static int chunk_pos(int r, int c) { return r * CH + (c ^ (r % CH)); }
  // 32-byte segment s of V row r sits at segment s ^ (r mod NSEG): the 16
  // rows one transposing read touches then spread evenly over the banks.
  __device__ static int vseg(int r, int s) { return s ^ (r & (NSEG - 1)); }
};

// IEEE maximum (gfx950 v_maximum3_f32): unlike fmaxf it needs no quieting
// of its inputs, so a max over raw MFMA results costs one instruction per
// two values. Masked keys are -inf by selection, never NaN, so the rows it
// sees hold no NaN unless the inputs do.
__device__ __forceinline__ float max_nq(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float row16_max_nq(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_nq(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row32_max_nq(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_nq(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum of a lane's NCT x 4 weights as a balanced tree, in a fixed order.
template <int NCT>
__device__ __forceinline__ float tree_sum(const float (&p)[NCT][4]) {
  float q[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) q[ct] = (p[ct][0] + p[ct][1]) + (p[ct][2] + p[ct][3]);
#pragma unroll
  for (int w = 1; w < NCT; w *= 2)
#pragma unroll
    for (int ct = 0; ct + w < NCT; ct += 2 * w) q[ct] += q[ct + w];
  return q[0];
}

template <int D, int G, int KT>
__global__ __launch_bounds__(256, KT == 32 ? 3 : 2) void prefill_attn_dma_kernel(PrefillParams P) {
  static_assert(KT == 32 || KT == 64, "key tile of 32 or 64");
  using L = PfDma<D, KT>;
  constexpr int QT = kPRows / G;   // query tokens per workgroup
  constexpr int NDT = D / 16;      // output column tiles (head dims)
  constexpr int NKS = D / 32;      // k-steps of the logits
  constexpr int NCT = KT / 16;     // 16-key column tiles of the logits
  constexpr int NST = KT / 32;     // k-steps of the PV product
  __shared__ __align__(16) char Ks0[L::KB];
  __shared__ __align__(16) char Ks1[L::KB];
  __shared__ __align__(16) char Vs0[L::KB];
  __shared__ __align__(16) char Vs1[L::KB];
  __shared__ int32_t s_tab[kPfTabLds];

  // Workgroups go to the 8 XCDs round-robin in id order. Renumber them so
  // the query tiles of one (request, kv-head) run on one XCD, back to back:
  // its K/V tiles, re-read by every query tile, then stay in that XCD's L2.
  // Within a unit, heavy (late) tiles first.
  const int ntq = (P.max_q_len + QT - 1) / QT;
  int r, h, qt;
  {
    const uint32_t W = gridDim.x * gridDim.y * gridDim.z;
    const uint32_t w = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const uint32_t x = w & 7, q8 = W >> 3, rem = W & 7;
    const uint32_t L = x * q8 + min(x, rem) + (w >> 3);
    const uint32_t unit = L / (uint32_t)ntq;
    qt = ntq - 1 - (int)(L - unit * (uint32_t)ntq);
    h = (int)(unit % (uint32_t)P.h_kv);
    r = (int)(unit / (uint32_t)P.h_kv);
  }
  int c0, qlen, ctx;
  if (!chunk_of(P, r, &c0, &qlen, &ctx, qt == ntq - 1)) return;
  const int q0 = qt * QT;
  if (q0 >= qlen) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, cl = lane & 15;
  const int q_last = min(qlen, q0 + QT) - 1;
  const int n_keys = ctx + q_last + 1;             // keys any row of the tile may see
  const int ntiles = (n_keys + KT - 1) / KT;
  const int32_t* tab = P.tables + (int64_t)r * P.table_stride;
  const bf16_t* kcache = reinterpret_cast<const bf16_t*>(P.kc) + P.kv_layer_off;
  const bf16_t* vcache = reinterpret_cast<const bf16_t*>(P.vc) + P.kv_layer_off;
  const int h_q = P.h_kv * G;

  int gi_of[2], ti0_of[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int row0 = (2 * wv + k) * 16;
    gi_of[k] = row0 / QT;
    ti0_of[k] = row0 % QT;
  }
  bf16x8_t qop[2][NKS];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = min(q0 + ti0_of[k] + cl, qlen - 1);  // rows past the chunk are discarded
    const bf16_t* qr = reinterpret_cast<const bf16_t*>(P.q) +
                       ((int64_t)(c0 + i) * h_q + h * G + gi_of[k]) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qop[k][ks] = __builtin_bit_cast(bf16x8_t, ld16(qr + ks * 32 + q * 8));
  }

  {  // block ids of the keys this workgroup reads (chunk_of bounds them by table_stride)
    const int npg = (n_keys + P.b - 1) >> P.log2b;
    for (int i = tid; i < npg; i += 256) s_tab[i] = tab[i];
  }
  __syncthreads();

  bool bad = false;  // a needed tile sits on an out-of-range block id
  // Byte offsets, inside a tile of K (V) rows, of the 16-byte chunk this
  // lane copies in each of its KI copies: LDS chunk p holds row p / CH and,
  // for K, chunk (p % CH) ^ (row % CH); for V, the chunk whose 32-byte
  // segment vseg places there.
  // unsigned: the copies then take a scalar base plus a 32-bit lane offset
  uint32_t koff[L::KI], voff[L::KI];
  int vrow[L::KI];
#pragma unroll
  for (int i = 0; i < L::KI; ++i) {
    const int pidx = (wv * L::KI + i) * 64 + lane;
    const int kr = pidx / L::CH, pc = pidx % L::CH;
    koff[i] = (kr * D + (pc ^ (kr % L::CH)) * 8) * 2;
    voff[i] = kr * D * 2 + L::vseg(kr, pc >> 1) * 32 + (pc & 1) * 16;
    vrow[i] = kr;
  }
  // Copy tile t into (Kb, Vb), 16 bytes per lane and copy: K rows whole, V
  // rows of existing keys; a bad block or keys past n_keys are written as
  // zeros instead (their weights are 0, and 0 x garbage must not reach O).
  auto issue = [&](int t, char* Kb, char* Vb) __attribute__((always_inline)) {
    const int page = s_tab[(t * KT) >> P.log2b];
    const bool ok = page >= 0 && page < P.num_blocks;
    bad |= !ok;
    const int row0 = ((page * P.h_kv + h) * P.b) + ((t * KT) & (P.b - 1));
    if (ok) {
      const char* kt = reinterpret_cast<const char*>(kcache + (int64_t)row0 * D);
      const char* vt = reinterpret_cast<const char*>(vcache + (int64_t)row0 * D);
#pragma unroll
      for (int i = 0; i < L::KI; ++i)
        __builtin_amdgcn_global_load_lds((gbl_void_ptr)(kt + koff[i]),
                                         (lds_void_ptr)(Kb + (wv * L::KI + i) * 1024), 16, 0, 0);
      if (t * KT + KT <= n_keys) {  // every row of the tile exists
#pragma unroll
        for (int i = 0; i < L::KI; ++i)
          __builtin_amdgcn_global_load_lds((gbl_void_ptr)(vt + voff[i]),
                                           (lds_void_ptr)(Vb + (wv * L::KI + i) * 1024), 16, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < L::KI; ++i) {
          if (t * KT + vrow[i] < n_keys)
            __builtin_amdgcn_global_load_lds((gbl_void_ptr)(vt + voff[i]),
                                             (lds_void_ptr)(Vb + (wv * L::KI + i) * 1024), 16, 0, 0);
          else
            *reinterpret_cast<uint4*>(Vb + ((wv * L::KI + i) * 64 + lane) * 16) = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < L::KI; ++i) {
        *reinterpret_cast<uint4*>(Kb + ((wv * L::KI + i) * 64 + lane) * 16) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(Vb + ((wv * L::KI + i) * 64 + lane) * 16) = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  floatx4 o[2][NDT];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[k][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-1.0e30f, -1.0e30f}, l[2] = {0.f, 0.f};
  int qpos[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) qpos[k] = ctx + q0 + ti0_of[k] + cl;  // this lane's query position
  const int vrr = 4 * q + (cl >> 2);                                  // Vᵀ read, key row 4q + cl/4
  const int vbase = vrr * L::VS + 8 * (cl & 3);
  // This lane's Vᵀ read offset within a V tile, per 16 head dims dt. Kept
  // opaque, so that each read adds the tile's LDS base (a constant of the
  // unrolled loop) as its immediate offset instead of a VALU add per read.
  uint32_t vro[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    vro[dt] = (uint32_t)(vbase + 32 * L::vseg(vrr, dt));
    asm volatile("" : "+v"(vro[dt]));
  }

  auto tile = [&](int t, const char* Kb, const char* Vb, char* Kn, char* Vn) __attribute__((always_inline)) {
    if (t + 1 < ntiles) issue(t + 1, Kn, Vn);  // in flight while this tile is used
    const bool diag = t * KT + KT - 1 > ctx + q0;  // some key may follow some query
    bf16x8_t pop[2][NST];
    floatx4 sk[2][NCT];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) sk[k][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const bf16x8_t kop = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(Kb + L::chunk_pos(ct * 16 + cl, ks * 4 + q) * 16));
        sk[0][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[0][ks], sk[0][ct], 0, 0, 0);
        sk[1][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[1][ks], sk[1][ct], 0, 0, 0);
      }
    // The softmax phase runs at raised wave priority, so the arbiter favours
    // a wavefront's VALU stretch over the other wavefront's MFMA stretch
    // (measured ~2% faster; raising it for the MFMA phases instead measured
    // ~2% slower).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      floatx4 (&s)[NCT] = sk[k];
      if (diag) {  // one branch, taken on the last tile or few only
        const int lim = qpos[k] - t * KT - 4 * q;  // last visible key offset
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (ct * 16 + v > lim) s[ct][v] = -INFINITY;
      }
      // weights against the running maximum as it stands
      float p[NCT][4];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v) p[ct][v] = __builtin_amdgcn_exp2f(fmaf(s[ct][v], P.qk_scale, -m[k]));
      // a tree (depth log2 of the weights), not a chain: the compare that
      // follows waits on it
      float ps = tree_sum<NCT>(p);
      if (__builtin_amdgcn_read_exec() & __ballot(!(ps <= psum_cap(4 * NCT)))) {
        // some weight too large (the first tile, whose running maximum is
        // -1e30, or a new maximum; NaN lands here too): the rows' maxima,
        // the rescale, and the weights again
        float mx = -INFINITY;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int v = 0; v < 4; v += 2) mx = max_nq(mx, max_nq(s[ct][v], s[ct][v + 1]));
        mx = row32_max_nq(row16_max_nq(mx));
        mx *= P.qk_scale;
        const float mn = fmaxf(m[k], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[k] - mn);
        m[k] = mn;
        l[k] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[k][dt] *= alpha;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int v = 0; v < 4; ++v) p[ct][v] = __builtin_amdgcn_exp2f(fmaf(s[ct][v], P.qk_scale, -m[k]));
        ps = tree_sum<NCT>(p);
      }
      l[k] += ps;
      // P operands: k-step st holds keys {32st + 4q + v} and {32st + 16 + 4q + v}
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        b2 x0 = __builtin_convertvector(f2{p[2 * st][0], p[2 * st][1]}, b2);
        b2 x1 = __builtin_convertvector(f2{p[2 * st][2], p[2 * st][3]}, b2);
        b2 x2 = __builtin_convertvector(f2{p[2 * st + 1][0], p[2 * st + 1][1]}, b2);
        b2 x3 = __builtin_convertvector(f2{p[2 * st + 1][2], p[2 * st + 1][3]}, b2);
        const uint4 u = make_uint4(__builtin_bit_cast(uint32_t, x0), __builtin_bit_cast(uint32_t, x1),
                                   __builtin_bit_cast(uint32_t, x2), __builtin_bit_cast(uint32_t, x3));
        pop[k][st] = __builtin_bit_cast(bf16x8_t, u);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // Oᵀ += Vᵀ Pᵀ: A = Vᵀ rows d = 16dt + cl from two transposing reads
    // (keys 32st + 4q + 0..3 and 32st + 16 + 4q + 0..3).
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const char* va = Vb + 32 * st * L::VS + vro[dt];  // rows + 32st keep vseg
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(va));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(va + 16 * L::VS));
        typedef short v8i16_t __attribute__((ext_vector_type(8)));
        const v8i16_t lh = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, lh);
#pragma unroll
        for (int k = 0; k < 2; ++k)
          o[k][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[k][st], o[k][dt], 0, 0, 0);
      }
    }
    __syncthreads();  // tile t + 1 has landed; every wavefront is done with this one
  };

  issue(0, Ks0, Vs0);
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    tile(t, Ks0, Vs0, Ks1, Vs1);
    if (t + 1 < ntiles) tile(t + 1, Ks1, Vs1, Ks0, Vs0);
  }

  if (bad) flag_error(P.err, ZP_DEVERR_BLOCK_ID);
  // Finish: the four lane groups hold partial sums of each query's weights.
  const int last = ctx + qlen - 1;
  bf16_t* out = reinterpret_cast<bf16_t*>(P.out);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float lt = xor32_sum(xor16_sum(l[k]));
    const int i = q0 + ti0_of[k] + cl;
    if (i >= qlen) continue;
    const float inv = 1.0f / lt;
    bf16_t* orow = out + ((int64_t)(c0 + i) * h_q + h * G + gi_of[k]) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint32_t w0 = uint32_t(f32_to_bf16(o[k][dt][0] * inv)) | (uint32_t(f32_to_bf16(o[k][dt][1] * inv)) << 16);
      const uint32_t w1 = uint32_t(f32_to_bf16(o[k][dt][2] * inv)) | (uint32_t(f32_to_bf16(o[k][dt][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(orow + dt * 16 + 4 * q) = make_uint2(w0, w1);
    }
    if (q == 0) emit_lse(P, r, c0, i, ctx + i, last, h, G, gi_of[k], (m[k] + log2f(lt)) * kLn2);
  }
}

// ---------------------------------------------------------------------------
// 2b. Any dtype: one workgroup per (token, kv-head, request), decode-style.
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void prefill_simple_kernel(PrefillParams P) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPR = D / EPL;    // lanes per key row
  constexpr int RPW = 64 / LPR;   // key rows per wavefront step
  __shared__ float sm_m[4 * RPW][G], sm_l[4 * RPW][G];
  __shared__ float sm_o[4 * RPW][G][D];
  const int r = blockIdx.z, h = blockIdx.y, i = blockIdx.x;
  int c0, qlen, ctx;
  if (!chunk_of(P, r, &c0, &qlen, &ctx, blockIdx.x == 0) || i >= qlen) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int grp = wv * RPW + lane / LPR, sub = lane % LPR;  // row group, lane in row
  const int pos = ctx + i;
  const int32_t* tab = P.tables + (int64_t)r * P.table_stride;
  const T* kcache = reinterpret_cast<const T*>(P.kc) + P.kv_layer_off;
  const T* vcache = reinterpret_cast<const T*>(P.vc) + P.kv_layer_off;
  const int h_q = P.h_kv * G;
  float qv[G][EPL];
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
    Vec16<T>::unpack(ld16(reinterpret_cast<const T*>(P.q) + ((int64_t)(c0 + i) * h_q + h * G + gi) * D + sub * EPL), qv[gi]);
  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    m[gi] = -1.0e30f;
    l[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[gi][e] = 0.f;
  }
  for (int t = grp; t <= pos; t += 4 * RPW) {
    const int page = tab[t >> P.log2b];
    if (page < 0 || page >= P.num_blocks) {
      if (sub == 0) flag_error(P.err, ZP_DEVERR_BLOCK_ID);
      continue;
    }
    const int64_t off = (((int64_t)page * P.h_kv + h) * P.b + (t & (P.b - 1))) * D + sub * EPL;
    float kf[EPL], vf[EPL];
    Vec16<T>::unpack(ld16(kcache + off), kf);
    Vec16<T>::unpack(ld16(vcache + off), vf);
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s = fmaf(qv[gi][e], kf[e], s);
      s = group_sum<LPR>(s) * P.qk_scale;
      const float mn = fmaxf(m[gi], s);
      const float a = exp2f(m[gi] - mn), pw = exp2f(s - mn);
      l[gi] = l[gi] * a + pw;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[gi][e] = fmaf(pw, vf[e], o[gi][e] * a);
      m[gi] = mn;
    }
  }
  if (sub == 0) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) { sm_m[grp][gi] = m[gi]; sm_l[grp][gi] = l[gi]; }
  }
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm_o[grp][gi][sub * EPL + e] = o[gi][e];
  __syncthreads();
  const int last = ctx + qlen - 1;
  T* out = reinterpret_cast<T*>(P.out);
  for (int x = tid; x < G * D; x += 256) {
    const int gi = x / D, e = x % D;
    float M = -1.0e30f;
    for (int g2 = 0; g2 < 4 * RPW; ++g2) M = fmaxf(M, sm_m[g2][gi]);
    float Ls = 0.f, O = 0.f;
    for (int g2 = 0; g2 < 4 * RPW; ++g2) {
      const float sc = exp2f(sm_m[g2][gi] - M);
      Ls += sm_l[g2][gi] * sc;
      O += sm_o[g2][gi][e] * sc;
    }
    out[((int64_t)(c0 + i) * h_q + h * G + gi) * D + e] = from_f32<T>(O / Ls);
    if (e == 0) emit_lse(P, r, c0, i, pos, last, h, G, gi, (M + log2f(Ls)) * kLn2);
  }
}

template <typename T, int D, int G>
static void launch_prefill(const PrefillParams& P, hipStream_t s) {
  dim3 ga((P.max_q_len + 63) / 64, P.h_kv, P.nreq);
  hipLaunchKernelGGL((prefill_append_kernel<T, D, G>), ga, dim3(256), 0, s, P);
  if constexpr (sizeof(T) == 2) {
    constexpr int QT = kPRows / G;
    dim3 g((P.max_q_len + QT - 1) / QT, P.h_kv, P.nreq);
    if (P.b >= kPfDmaKT && P.table_stride <= kPfTabLds)
      hipLaunchKernelGGL((prefill_attn_dma_kernel<D, G, kPfDmaKT>), g, dim3(256), 0, s, P);
    else
      hipLaunchKernelGGL((prefill_attn_kernel<D, G>), g, dim3(256), 0, s, P);
  } else {
    dim3 g(P.max_q_len, P.h_kv, P.nreq);
    hipLaunchKernelGGL((prefill_simple_kernel<T, D, G>), g, dim3(256), 0, s, P);
  }
}

template <typename T, int D>
static void prefill_group(int g, const PrefillParams& P, hipStream_t s) {
  switch (g) {
    case 1: launch_prefill<T, D, 1>(P, s); break;
    case 2: launch_prefill<T, D, 2>(P, s); break;
    case 4: launch_prefill<T, D, 4>(P, s); break;
    default: launch_prefill<T, D, 8>(P, s); break;
  }
}

}  // namespace zp

using namespace zp;

extern "C" size_t zp_prefill_workspace_size(const zp_geom* geom, int32_t nreq) {
  if (validate_geom(geom, "zp_prefill_workspace_size") != ZP_OK || nreq < 0) return 0;
  return kWsHeader;
}

extern "C" zp_status zp_paged_prefill(const zp_geom* geom, const zp_cache* cache, int32_t layer,
                                      int32_t nreq, const void* q, const void* k_new,
                                      const void* v_new, const int32_t* cu_seqlens,
                                      const int32_t* ctx_lens, int32_t max_q_len,
                                      const int32_t* block_tables, int32_t table_stride,
                                      const int32_t* qslot, void* out, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  zp_status st = validate_geom(geom, "zp_paged_prefill");
  if (st != ZP_OK) return st;
  if (!cache || !cache->k || !cache->v) return fail(ZP_EINVAL, "zp_paged_prefill: cache K/V NULL");
  if (layer < 0 || layer >= geom->num_layers)
    return fail(ZP_EINVAL, "zp_paged_prefill: layer %d out of range", layer);
  if (nreq < 0 || max_q_len < 0 || table_stride <= 0)
    return fail(ZP_EINVAL, "zp_paged_prefill: bad nreq/max_q_len/table_stride");
  if (nreq == 0 || max_q_len == 0) return ZP_OK;
  if (nreq > 65535 || max_q_len > (1 << 24))
    return fail(ZP_EINVAL, "zp_paged_prefill: nreq must be <= 65535 and max_q_len <= 2^24");
  if (!q || !k_new || !v_new || !cu_seqlens || !ctx_lens || !block_tables || !out || !workspace)
    return fail(ZP_EINVAL, "zp_paged_prefill: NULL buffer");
  if (qslot && !cache->qwin) return fail(ZP_EINVAL, "zp_paged_prefill: qslot given but qwin NULL");
  if (workspace_bytes < kWsHeader)
    return fail(ZP_EINVAL, "zp_paged_prefill: workspace %zu bytes, need %zu", workspace_bytes,
                kWsHeader);

  PrefillParams P{};
  P.q = q; P.k_new = k_new; P.v_new = v_new;
  P.kc = cache->k; P.vc = cache->v; P.qwin = cache->qwin; P.qwin_lse = cache->qwin_lse;
  P.cu = cu_seqlens; P.ctx = ctx_lens; P.tables = block_tables; P.qslot = qslot;
  P.out = out; P.lse = lse;
  P.err = static_cast<uint32_t*>(workspace);
  const int64_t d = geom->head_dim;
  P.kv_layer_off = int64_t(layer) * geom->num_blocks * geom->num_kv_heads * geom->block_size * d;
  P.qwin_layer_off = int64_t(layer) * geom->max_slots * geom->num_q_heads * geom->window * d;
  P.qlse_layer_off = int64_t(layer) * geom->max_slots * geom->num_q_heads * geom->window;
  P.nreq = nreq; P.table_stride = table_stride; P.num_blocks = geom->num_blocks;
  P.b = geom->block_size; P.h_kv = geom->num_kv_heads; P.w = geom->window;
  P.max_slots = geom->max_slots; P.max_q_len = max_q_len;
  P.log2b = __builtin_ctz(unsigned(geom->block_size));
  P.qk_scale = kLog2e / std::sqrt(float(d));

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int g = group_size(geom);
  if (geom->dtype == ZP_DTYPE_BF16) {
    if (d == 128) prefill_group<bf16_t, 128>(g, P, s);
    else prefill_group<bf16_t, 64>(g, P, s);
  } else {
    if (d == 128) prefill_group<float, 128>(g, P, s);
    else prefill_group<float, 64>(g, P, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZP_EHIP, "zp_paged_prefill: launch failed: %s", hipGetErrorString(e));
  return ZP_OK;
}
