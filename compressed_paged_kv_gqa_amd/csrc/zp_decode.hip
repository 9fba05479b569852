// Paged grouped-query decode attention for gfx950 (one layer, one step).
//
// Zipage (arXiv 2603.08743): Sec. 3 (K/V in fixed-size blocks addressed
// through per-request block tables), Sec. 4.2 (the query of each of the last
// w slots of a block is kept in the query cache), Sec. 6 (eviction does not
// change the attention forward: it is softmax attention over whatever tokens
// are resident).
//
// Design (HBM-bound, 4 FLOP per byte, so no MFMA):
//  * one workgroup of 4 wavefronts per (split, kv-head, sequence); a split is
//    a contiguous token range, so every K/V byte of the sequence is read once
//    for all g query heads of the kv-head;
//  * a token row of d elements is read by d*sizeof(T)/16 lanes with 16-byte
//    loads, so one wavefront load instruction covers 1 KiB of contiguous
//    K (or V) and the head-major page layout keeps the stream sequential;
//  * q.k partial dot products are reduced inside each row group with DPP
//    (no LDS; for bf16, d = 128, g = 4 one transposing reduction of the 16
//    (head, row) products), softmax is online in exp2 form per chunk;
//  * a sequence is split over several workgroups only when the (sequence,
//    kv-head) items alone cannot fill the GPU; then a second small kernel
//    merges the split partials (max, sum, unnormalised output). A device-wide
//    fence per workgroup (to merge in the same launch) costs far more than
//    that extra launch on this chip (measured);
//  * the block ids of a split are requested together with the sequence
//    length; the first 64 sit one per lane in every wavefront (the first
//    chunk's loads go out before any barrier), the rest are staged in LDS, so
//    no K/V load in the loop waits behind a block-table load;
//  * K/V chunks come through buffer loads; a chunk past the end gets an
//    empty range (zeros, no memory read), so the next chunk's loads are
//    issued unconditionally and the waits cover only the chunk in use;
//  * the token being decoded is written to its slot, before the chunk loop,
//    by the one wavefront that reads that chunk: no other workgroup reads
//    that slot, so append and attention need no extra launch.
#include <cmath>
#include <mutex>

#include "zp_device.h"
#include "zp_internal.h"

namespace zp {

struct DecodeParams {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* kc;
  void* vc;
  void* qwin;
  float* qwin_lse;
  const int32_t* tables;
  const int32_t* seq_lens;
  const int32_t* qslot;
  void* out;
  float* lse;
  float* part;        // [batch][h_kv][max_splits][G][D + 2]
  uint32_t* err;
  int64_t kv_layer_off;    // element offset of the layer in K / V
  int64_t qwin_layer_off;  // element offset of the layer in Qwin
  int64_t qlse_layer_off;  // element offset of the layer in the Qwin LSE table
  int32_t table_stride, num_blocks, b, h_kv, w, max_slots;
  int32_t split_tokens, max_splits, max_seq_len, log2b, waves;
  float qk_scale;  // log2(e) / sqrt(d)
};

template <typename T, int D, int G>
struct DecodeCfg {
  static constexpr int EPL = Vec16<T>::N;  // elements per lane per 16-byte load
  static constexpr int LPR = D / EPL;      // lanes per token row
  static constexpr int RPW = 64 / LPR;     // token rows per wavefront load
  static constexpr int CHUNK = 16;         // tokens per wavefront chunk (never crosses a block)
  static constexpr int U = CHUNK / RPW;    // row loads per lane per chunk (K and V each)
  // waves per SIMD the register budget is sized for (no spills)
  static constexpr int MIN_WAVES = decode_waves_per_simd(sizeof(T), D, G);
};

// Query registers of one lane: its EPL dims of the g query heads.
template <typename T, int G>
struct QRegs;

template <int G>
struct QRegs<bf16_t, G> {
  uint32_t w[G][4];  // 8 bf16 per head, packed in pairs
  __device__ void load(const bf16_t* q, int64_t head_stride) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 v = ld16(q + h * head_stride);
      w[h][0] = v.x; w[h][1] = v.y; w[h][2] = v.z; w[h][3] = v.w;
    }
  }
  // q_h . k over this lane's 8 dims (bf16 pairs, fp32 accumulation)
  __device__ float dot(int h, const uint4& k) const {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    float a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w[h][0]),
                                              __builtin_bit_cast(bf2, k.x), 0.f, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w[h][1]),
                                        __builtin_bit_cast(bf2, k.y), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w[h][2]),
                                        __builtin_bit_cast(bf2, k.z), a, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, w[h][3]),
                                           __builtin_bit_cast(bf2, k.w), a, false);
  }
};

template <int G>
struct QRegs<float, G> {
  float w[G][4];
  __device__ void load(const float* q, int64_t head_stride) {
#pragma unroll
    for (int h = 0; h < G; ++h) Vec16<float>::unpack(ld16(q + h * head_stride), w[h]);
  }
  __device__ float dot(int h, const uint4& k) const {
    float a = w[h][0] * __uint_as_float(k.x);
    a = fmaf(w[h][1], __uint_as_float(k.y), a);
    a = fmaf(w[h][2], __uint_as_float(k.z), a);
    return fmaf(w[h][3], __uint_as_float(k.w), a);
  }
};

// Online-softmax state of one lane for its token-row group. Rescaling is
// lazy: a chunk rescales only when its maximum exceeds the running one by
// more than kLazy (log2 units), so p = exp2(s - m) stays below 2^kLazy.
constexpr float kLazy = 8.0f;
// Upper bound on the blocks one split covers (decode_launch_shape keeps
// split_tokens <= kMaxSplitPages * block_size).
constexpr int kMaxSplitPages = 1024;
constexpr float kNoMax = -1.0e30f;  // finite "nothing seen yet"

// Window row of the token at position n - 1 of sequence `seq` (its slot in
// the query cache), or -1 when the token is not in the final w slots of its
// block or no valid query-cache slot is given.
__device__ __forceinline__ int window_row_of(const DecodeParams& P, int seq, int n, int* slot) {
  if (!P.qslot) return -1;
  const int off = (n - 1) % P.b;
  const int s = P.qslot[seq];
  if (off < P.b - P.w || s < 0 || s >= P.max_slots) return -1;
  *slot = s;
  return off - (P.b - P.w);
}

// WAVES wavefronts per workgroup (one workgroup per (split, kv-head,
// sequence)); they take the chunks of the split in turn and are merged in
// LDS at the end.
template <typename T, int D, int G, int WAVES>
__global__ __launch_bounds__(64 * WAVES, (DecodeCfg<T, D, G>::MIN_WAVES)) void paged_decode_kernel(
    DecodeParams P) {
  using C = DecodeCfg<T, D, G>;
  constexpr int EPL = C::EPL, LPR = C::LPR, RPW = C::RPW, U = C::U, CHUNK = C::CHUNK;
  constexpr int NT = 64 * WAVES;  // threads

  __shared__ float sm_m[WAVES][G];
  __shared__ float sm_l[WAVES][G];
  __shared__ float sm_o[WAVES][G][D];
  __shared__ int sm_pages[kMaxSplitPages];

  const int split = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int32_t* tab = P.tables + (int64_t)seq * P.table_stride;
  // Block ids of this split, requested before the sequence length is read:
  // from the split's first block as many as a split can span (within the
  // table row), so the table load does not wait for the length.
  const int t0 = split * P.split_tokens;
  const int pg0 = t0 >> P.log2b;
  const int span = min(min(P.table_stride - pg0, ((P.split_tokens - 1) >> P.log2b) + 2), kMaxSplitPages);
  const int n = P.seq_lens[seq];
  const int pg_first = tid < span ? tab[pg0 + tid] : 0;  // in flight with the length
  const int pg_lane = lane < span ? tab[pg0 + lane] : 0;  // the first 64, in every wavefront
  // This lane's 16 bytes of the decoded token's k and v (one of the
  // wavefronts appends them below).
  const int64_t new_off = ((int64_t)seq * P.h_kv + kvh) * D + (lane % (D / Vec16<T>::N)) * Vec16<T>::N;
  const uint4 k_tok = ld16(reinterpret_cast<const T*>(P.k_new) + new_off);
  const uint4 v_tok = ld16(reinterpret_cast<const T*>(P.v_new) + new_off);
  if (n <= 0) return;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront index, made scalar
  const int h_q = P.h_kv * G;
  const int64_t out_row = (int64_t)seq * h_q + (int64_t)kvh * G;  // first head of the group

  if (n > P.max_seq_len || n > (int64_t)P.table_stride * P.b) {
    // The launch does not cover this row: report, poison its outputs.
    if (split == 0) {
      if (tid == 0) flag_error(P.err, ZP_DEVERR_SEQ_LEN);
      T* out = reinterpret_cast<T*>(P.out);
      for (int i = tid; i < G * D; i += NT) out[out_row * D + i] = from_f32<T>(NAN);
      if (P.lse && tid < G) P.lse[out_row + tid] = NAN;
    }
    return;
  }
  const int nsplit = (n + P.split_tokens - 1) / P.split_tokens;
  if (split >= nsplit) return;
  const int t1 = min(n, t0 + P.split_tokens);
  const int row = lane / LPR;
  const int sub = lane % LPR;
  const int b = P.b;
  T* kc = reinterpret_cast<T*>(P.kc) + P.kv_layer_off;
  T* vc = reinterpret_cast<T*>(P.vc) + P.kv_layer_off;
  const int64_t lane_off = (int64_t)kvh * b * D + (int64_t)row * D + sub * EPL;  // within a page
  const int64_t page_elems = (int64_t)P.h_kv * b * D;

  QRegs<T, G> q;
  q.load(reinterpret_cast<const T*>(P.q) + out_row * D + sub * EPL, D);

  const int npg = ((t1 - 1) >> P.log2b) - pg0 + 1;  // block ids the split uses (<= span)
  if (tid < span) sm_pages[tid] = pg_first;
  for (int i = tid + NT; i < npg; i += NT) sm_pages[i] = tab[pg0 + i];
  // (LDS copy visible after the barrier below, which follows the first
  // chunk's loads; until then ids come from pv.)

  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNoMax;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
  }
  // bf16 rows of 16 lanes carrying g * U = 16 (head, row) dot products per
  // chunk take the transposing reduction (see process); lane sub then owns
  // (head sub / U, row sub % U): its running max mj = m[sub / U] and its
  // weight sum lacc.
  constexpr bool kTR = sizeof(T) == 2 && LPR == 16 && G * U == 16;
  float lacc = 0.f, mj = kNoMax;

  const int nchunks = (t1 - t0 + CHUNK - 1) / CHUNK;
  // The first 64 block ids also sit one per lane: a chunk takes its id with
  // one lane read (no LDS access, no address register); later ones come from
  // the LDS copy.
  const int pv = lane < npg ? pg_lane : -1;
  auto page_of = [&](int bi) __attribute__((always_inline)) -> int {
    return bi < 64 ? __builtin_amdgcn_readlane(pv, bi) : __builtin_amdgcn_readfirstlane(sm_pages[bi]);
  };

  // Element offset of this lane's row 0 in chunk c, or -1 for a bad block id.
  auto chunk_offset = [&](int c) -> int64_t {
    const int base = t0 + c * CHUNK;
    const int page = page_of((base >> P.log2b) - pg0);
    if (page < 0 || page >= P.num_blocks) return -1;
    return (int64_t)page * page_elems + lane_off + (int64_t)(base & (b - 1)) * D;
  };
  // Chunk c through buffer loads whose range is the chunk's token rows in
  // its (block, kv-head) slice of K (or V), up to the end of the split: the
  // slots after the sequence return zeros and are not read. A chunk past the
  // end, or on a bad block id, gets an empty range: its loads return zeros
  // and read no memory. So the next chunk's loads are issued unconditionally, and the
  // compiler's waits in the loop cover only the chunk in use. Returns 0, or
  // -1 for a bad block id (the chunk is then masked).
  const uint32_t lane_bytes = (uint32_t)((row * D + sub * EPL) * sizeof(T));
  auto load_chunk = [&](int c, uint4 (&kr)[U], uint4 (&vr)[U]) __attribute__((always_inline)) -> int64_t {
    int64_t first = 0;  // element offset of the chunk's first row
    int bytes = 0, bad = 0;
    if (c < nchunks) {
      const int base = t0 + c * CHUNK;
      const int page = page_of((base >> P.log2b) - pg0);
      if (page >= 0 && page < P.num_blocks) {
        first = (int64_t)page * page_elems + (int64_t)kvh * b * D + (int64_t)(base & (b - 1)) * D;
        bytes = min(t1 - base, CHUNK) * D * (int)sizeof(T);
      } else {
        bad = -1;
      }
    }
    const BufRsrc rk = make_rsrc(kc + first, bytes);
    const BufRsrc rv = make_rsrc(vc + first, bytes);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kr[u] = ldbuf16_nt(rk, lane_bytes + (uint32_t)(u * RPW * D * sizeof(T)));
      vr[u] = ldbuf16_nt(rv, lane_bytes + (uint32_t)(u * RPW * D * sizeof(T)));
    }
    return bad;
  };
  auto process = [&](int c, uint4 (&kr)[U], uint4 (&vr)[U], int64_t off) __attribute__((always_inline)) {
    const int base = t0 + c * CHUNK;
    if (off < 0 && lane == 0) flag_error(P.err, ZP_DEVERR_BLOCK_ID);
    // Raw q.k (unscaled); the 1/sqrt(d) * log2(e) factor enters the exp.
    float s[G][U];
    const float sc2 = P.qk_scale;
    if constexpr (kTR) {
      // The row group's 16 (head, row) dot products: one transposing sum
      // leaves (head sub / U, row sub % U) in lane sub; the chunk maximum of
      // a head is a max over its 4 lanes (one quad), the weight is one
      // exp2 per lane, and the 16 weights are broadcast back to every lane
      // of the row group for o += p v. l accumulates the lane's own weights
      // (lacc) and is summed over each quad after the last chunk.
      float part[G * U];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int h = 0; h < G; ++h) part[h * U + u] = q.dot(h, kr[u]);
      float sj = row_transpose_sum16(part, sub);
      if (base + CHUNK > t1 || off < 0) {
        // Masked rows (see below): weight exactly 0, V zeroed.
        if (!(off >= 0 && base + (sub % U) * RPW + row < t1)) sj = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (!(off >= 0 && base + u * RPW + row < t1)) vr[u] = make_uint4(0u, 0u, 0u, 0u);
      }
      float cq = fmaxf(sj, dpp_z<DPP_QUAD_XOR1>(sj));
      cq = fmaxf(cq, dpp_z<DPP_QUAD_XOR2>(cq));
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float cm = bcast_row_lane(cq, 4 * h) * sc2;  // head h's chunk max
        if (cm > m[h] + kLazy) {
          const float alpha = __builtin_amdgcn_exp2f(m[h] - cm);
          if (sub / U == h) {
            lacc *= alpha;
            mj = cm;
          }
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
          m[h] = cm;
        }
      }
      const float pj = __builtin_amdgcn_exp2f(fmaf(sj, sc2, -mj));
      lacc += pj;
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int u = 0; u < U; ++u) s[h][u] = bcast_row_lane(pj, h * U + u);
    } else {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) s[h][u] = group_sum<LPR>(q.dot(h, kr[u]));
    if (base + CHUNK > t1 || off < 0) {
      // Masked rows: slots past the sequence (never written, may hold
      // anything, NaN included) or a bad block. Their weight is exactly 0
      // and their V is zeroed, so 0 * garbage never enters the sum.
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool valid = off >= 0 && base + u * RPW + row < t1;
#pragma unroll
        for (int h = 0; h < G; ++h) s[h][u] = valid ? s[h][u] : -INFINITY;
        if (!valid) vr[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float cm = s[h][0];
#pragma unroll
      for (int u = 1; u < U; ++u) cm = fmaxf(cm, s[h][u]);
      cm *= sc2;
      if (cm > m[h] + kLazy) {
        const float alpha = __builtin_amdgcn_exp2f(m[h] - cm);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
        m[h] = cm;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) s[h][u] = __builtin_amdgcn_exp2f(fmaf(s[h][u], sc2, -m[h]));  // p
    }
    }
    if constexpr (sizeof(T) == 2) {
      // o += p v over token pairs (u, u+1) with packed-bf16 dot products:
      // the weights enter the numerator rounded to bf16 (the normaliser l
      // keeps the fp32 values), V of the two tokens interleaved per
      // dimension with v_perm.
      typedef float f2 __attribute__((ext_vector_type(2)));
      typedef __bf16 b2 __attribute__((ext_vector_type(2)));
      if constexpr (!kTR) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int u = 0; u < U; ++u) l[h] += s[h][u];
      }
#pragma unroll
      for (int u = 0; u < U; u += 2) {
        b2 pp[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pp[h] = __builtin_convertvector(f2{s[h][u], s[h][u + 1]}, b2);
        const uint32_t a[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
        const uint32_t bb[4] = {vr[u + 1].x, vr[u + 1].y, vr[u + 1].z, vr[u + 1].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const b2 lo = __builtin_bit_cast(b2, __builtin_amdgcn_perm(bb[j], a[j], 0x05040100u));
          const b2 hi = __builtin_bit_cast(b2, __builtin_amdgcn_perm(bb[j], a[j], 0x07060302u));
#pragma unroll
          for (int h = 0; h < G; ++h) {
            o[h][2 * j] = __builtin_amdgcn_fdot2_f32_bf16(pp[h], lo, o[h][2 * j], false);
            o[h][2 * j + 1] = __builtin_amdgcn_fdot2_f32_bf16(pp[h], hi, o[h][2 * j + 1], false);
          }
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int u = 0; u < U; ++u) l[h] += s[h][u];
      // o += p v, one V row at a time (keeps few unpacked values live).
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float vf[EPL];
        Vec16<T>::unpack(vr[u], vf);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(s[h][u], vf[e], o[h][e]);
      }
    }
  };

  // The token being decoded goes to its slot first, written by the wavefront
  // whose chunk holds it; that wavefront reads it back with the rest of the
  // chunk, so the chunk loop carries no special case. The wait retires the
  // two stores before that chunk's loads are issued: ahead of the first
  // chunk's loads when the token's block id is among the first 64 (always
  // so when its chunk is a wavefront's first), else after the barrier.
  const bool tok_here = t0 <= n - 1 && n - 1 < t1 && ((n - 1 - t0) / CHUNK) % WAVES == wv;
  const bool tok_early = ((n - 1) >> P.log2b) - pg0 < 64;
  auto append_token = [&]() __attribute__((always_inline)) {
    const int r = (n - 1 - t0) % CHUNK;  // u * RPW + row of the token in its chunk
    const int64_t off = chunk_offset((n - 1 - t0) / CHUNK);
    if (off >= 0 && r % RPW == row) {
      const int64_t at = off + (int64_t)(r / RPW) * RPW * D;
      st16(kc + at, k_tok);
      st16(vc + at, v_tok);
    }
    __builtin_amdgcn_s_waitcnt(0);
  };
  if (tok_here && tok_early) append_token();

  // Chunks c = wv, wv + 4, ...; the next chunk's loads are issued before the
  // current chunk is processed (two register buffers). The first chunk's
  // loads go out before the barrier that publishes the LDS block ids.
  {
    uint4 ka[U], va[U], kb[U], vb[U];
    int c = wv;
    int64_t offa = load_chunk(c, ka, va), offb;
    __syncthreads();
    if (tok_here && !tok_early) append_token();
    while (c < nchunks) {
      offb = load_chunk(c + WAVES, kb, vb);
      process(c, ka, va, offa);
      c += WAVES;
      if (c >= nchunks) break;
      offa = load_chunk(c + WAVES, ka, va);
      process(c, kb, vb, offb);
      c += WAVES;
    }
  }

  if constexpr (kTR) {  // l of every head from its quad of lanes
    float lq = lacc + dpp_z<DPP_QUAD_XOR1>(lacc);
    lq += dpp_z<DPP_QUAD_XOR2>(lq);
#pragma unroll
    for (int h = 0; h < G; ++h) l[h] = bcast_row_lane(lq, 4 * h);
  }
  // Merge the token-row groups of the wavefront.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = across_groups_max<LPR>(m[h]);
    const float sc = __builtin_amdgcn_exp2f(m[h] - M);
    l[h] = across_groups_sum<LPR>(l[h] * sc);
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = across_groups_sum<LPR>(o[h][e] * sc);
    m[h] = M;
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wv][h][sub * EPL + e] = o[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_m[wv][h] = m[h];
      sm_l[wv][h] = l[h];
    }
  }
  __syncthreads();

  // Capture the window query (by the split that holds the new token).
  if (P.qslot && split == nsplit - 1) {
    const int pos = n - 1;
    const int off = pos % P.b;
    const int slot = P.qslot[seq];
    if (slot >= 0 && off >= P.b - P.w) {
      if (slot >= P.max_slots) {
        if (tid == 0) flag_error(P.err, ZP_DEVERR_SLOT);
      } else {
        const T* qp = reinterpret_cast<const T*>(P.q) + out_row * D;
        T* dst = reinterpret_cast<T*>(P.qwin) + P.qwin_layer_off +
                 (((int64_t)slot * P.h_kv + kvh) * G) * P.w * D + (int64_t)(off - (P.b - P.w)) * D;
        for (int i = tid; i < G * D; i += NT) {
          const int h = i / D, e = i % D;
          dst[(int64_t)h * P.w * D + e] = qp[i];
        }
      }
    }
  }

  // Combine the wavefronts: each thread owns (head, dim) pairs.
  constexpr int PAIRS = G * D;
  constexpr int PPT = (PAIRS + NT - 1) / NT;  // pairs per thread
  float Mw[PPT], Lw[PPT], Ow[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int i = tid + k * NT;
    Mw[k] = kNoMax; Lw[k] = 0.f; Ow[k] = 0.f;
    if (i < PAIRS) {
      const int h = i / D, e = i % D;
      float M = sm_m[0][h];
#pragma unroll
      for (int w2 = 1; w2 < WAVES; ++w2) M = fmaxf(M, sm_m[w2][h]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < WAVES; ++w2) {
        const float sc = __builtin_amdgcn_exp2f(sm_m[w2][h] - M);
        L += sm_l[w2][h] * sc;
        O += sm_o[w2][h][e] * sc;
      }
      Mw[k] = M; Lw[k] = L; Ow[k] = O;
    }
  }

  T* out = reinterpret_cast<T*>(P.out);
  if (nsplit == 1) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int i = tid + k * NT;
      if (i < PAIRS) {
        const int h = i / D, e = i % D;
        out[(out_row + h) * D + e] = from_f32<T>(Ow[k] / Lw[k]);
        if (e == 0) {
          const float lse_nat = (Mw[k] + log2f(Lw[k])) * kLn2;
          if (P.lse) P.lse[out_row + h] = lse_nat;
          int slot;
          const int u = P.qwin_lse ? window_row_of(P, seq, n, &slot) : -1;
          if (u >= 0)
            P.qwin_lse[P.qlse_layer_off + (((int64_t)slot * P.h_kv + kvh) * G + h) * P.w + u] = lse_nat;
        }
      }
    }
    return;
  }

  // Several splits: publish this split's partial; zp_decode_merge_kernel
  // combines them.
  const int64_t item = (int64_t)seq * P.h_kv + kvh;
  float* mypart = P.part + (item * P.max_splits + split) * G * (D + 2);
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int i = tid + k * NT;
    if (i < PAIRS) {
      const int h = i / D, e = i % D;
      mypart[h * (D + 2) + 2 + e] = Ow[k];
      if (e == 0) {
        mypart[h * (D + 2)] = Mw[k];
        mypart[h * (D + 2) + 1] = Lw[k];
      }
    }
  }
}

// Merges the split partials of every (sequence, kv-head) row that was split.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams P) {
  const int kvh = blockIdx.x, seq = blockIdx.y;
  const int n = P.seq_lens[seq];
  if (n <= 0 || n > P.max_seq_len || n > (int64_t)P.table_stride * P.b) return;
  const int nsplit = (n + P.split_tokens - 1) / P.split_tokens;
  if (nsplit <= 1) return;  // written directly by the decode kernel
  const int64_t item = (int64_t)seq * P.h_kv + kvh;
  const int64_t out_row = (int64_t)seq * P.h_kv * G + (int64_t)kvh * G;
  const float* parts = P.part + item * P.max_splits * G * (D + 2);
  T* out = reinterpret_cast<T*>(P.out);
  for (int i = threadIdx.x; i < G * D; i += 256) {
    const int h = i / D, e = i % D;
    // the splits' (max, sum, output) merged online in split order, four
    // splits' loads in flight at a time (two passes of single loads would
    // wait for each in turn)
    float M = kNoMax, L = 0.f, O = 0.f;
    auto merge = [&](float pm, float pl, float po) __attribute__((always_inline)) {
      const float mn = fmaxf(M, pm);
      const float a = __builtin_amdgcn_exp2f(M - mn), c = __builtin_amdgcn_exp2f(pm - mn);
      L = L * a + pl * c;
      O = O * a + po * c;
      M = mn;
    };
    int s2 = 0;
    for (; s2 + 4 <= nsplit; s2 += 4) {
      float pm[4], pl[4], po[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* pp = parts + ((s2 + j) * G + h) * (D + 2);
        pm[j] = pp[0];
        pl[j] = pp[1];
        po[j] = pp[2 + e];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) merge(pm[j], pl[j], po[j]);
    }
    for (; s2 < nsplit; ++s2) {
      const float* pp = parts + (s2 * G + h) * (D + 2);
      merge(pp[0], pp[1], pp[2 + e]);
    }
    out[(out_row + h) * D + e] = from_f32<T>(O / L);
    if (e == 0) {
      const float lse_nat = (M + log2f(L)) * kLn2;
      if (P.lse) P.lse[out_row + h] = lse_nat;
      int slot;
      const int u = P.qwin_lse ? window_row_of(P, seq, n, &slot) : -1;
      if (u >= 0)
        P.qwin_lse[P.qlse_layer_off + (((int64_t)slot * P.h_kv + kvh) * G + h) * P.w + u] = lse_nat;
    }
  }
}

template <typename T, int D, int G>
static void launch_decode(const DecodeParams& P, int batch, hipStream_t stream) {
  dim3 grid(P.max_splits, P.h_kv, batch);
  constexpr int MW = DecodeCfg<T, D, G>::MIN_WAVES;
  // the workgroup sizes decode_launch_shape picks from: 4 wavefronts, or a
  // whole CU's resident waves (small batches)
  if (P.waves == 4 * MW)
    hipLaunchKernelGGL((paged_decode_kernel<T, D, G, 4 * MW>), grid, dim3(256 * MW), 0, stream, P);
  else
    hipLaunchKernelGGL((paged_decode_kernel<T, D, G, 4>), grid, dim3(256), 0, stream, P);
  if (P.max_splits > 1)
    hipLaunchKernelGGL((decode_merge_kernel<T, D, G>), dim3(P.h_kv, batch), dim3(256), 0, stream,
                       P);
}

template <typename T, int D>
static void dispatch_group(int g, const DecodeParams& P, int batch, hipStream_t s) {
  switch (g) {
    case 1: launch_decode<T, D, 1>(P, batch, s); break;
    case 2: launch_decode<T, D, 2>(P, batch, s); break;
    case 4: launch_decode<T, D, 4>(P, batch, s); break;
    default: launch_decode<T, D, 8>(P, batch, s); break;
  }
}

static size_t decode_ws_layout(const zp_geom* g, int32_t batch, int32_t max_seq_len,
                               size_t* part_off, int32_t* split_tokens, int32_t* max_splits,
                               int32_t* waves) {
  int32_t wv = 4;
  const int32_t st = decode_launch_shape(g, batch, max_seq_len, &wv);
  if (waves) *waves = wv;
  const int32_t ms = std::max<int32_t>(1, (std::max<int32_t>(max_seq_len, 1) + st - 1) / st);
  const size_t items = size_t(batch) * g->num_kv_heads;
  const size_t p_off = kWsHeader;
  const size_t total = p_off + (ms > 1 ? items * ms * group_size(g) * (g->head_dim + 2) * sizeof(float) : 0);
  if (part_off) *part_off = p_off;
  if (split_tokens) *split_tokens = st;
  if (max_splits) *max_splits = ms;
  return total;
}

// Checks the arguments of a decode call and computes its launch shape and
// the bytes of split partials it needs. No HIP call.
static zp_status decode_prepare(const zp_geom* geom, const zp_cache* cache, int32_t layer,
                                int32_t batch, const void* q, const void* k_new,
                                const void* v_new, const int32_t* block_tables,
                                int32_t table_stride, const int32_t* seq_lens,
                                int32_t max_seq_len, const int32_t* qslot, void* out,
                                const char* who, size_t* need, size_t* p_off,
                                int32_t* split_tokens, int32_t* max_splits, int32_t* waves) {
  zp_status st = validate_geom(geom, who);
  if (st != ZP_OK) return st;
  if (!cache || !cache->k || !cache->v) return fail(ZP_EINVAL, "%s: cache K/V NULL", who);
  if (layer < 0 || layer >= geom->num_layers)
    return fail(ZP_EINVAL, "%s: layer %d out of range", who, layer);
  if (batch < 0 || table_stride <= 0 || max_seq_len < 0)
    return fail(ZP_EINVAL, "%s: bad batch/table_stride/max_seq_len", who);
  if (batch == 0) {
    *need = 0;
    return ZP_OK;
  }
  if (!q || !k_new || !v_new || !block_tables || !seq_lens || !out)
    return fail(ZP_EINVAL, "%s: NULL buffer", who);
  if (qslot && !cache->qwin) return fail(ZP_EINVAL, "%s: qslot given but qwin NULL", who);
  *need = decode_ws_layout(geom, batch, max_seq_len, p_off, split_tokens, max_splits, waves);
  return ZP_OK;
}

// Enqueues the decode kernels of one call; partials at `part`, device error
// bits OR-ed into *err (may be NULL: dropped).
static zp_status decode_enqueue(const zp_geom* geom, const zp_cache* cache, int32_t layer,
                                int32_t batch, const void* q, const void* k_new,
                                const void* v_new, const int32_t* block_tables,
                                int32_t table_stride, const int32_t* seq_lens,
                                int32_t max_seq_len, const int32_t* qslot, void* out, float* lse,
                                float* part, uint32_t* err, int32_t split_tokens,
                                int32_t max_splits, int32_t waves, void* stream,
                                const char* who) {
  DecodeParams P{};
  P.q = q; P.k_new = k_new; P.v_new = v_new;
  P.kc = cache->k; P.vc = cache->v; P.qwin = cache->qwin;
  P.qwin_lse = qslot ? cache->qwin_lse : nullptr;
  P.tables = block_tables; P.seq_lens = seq_lens; P.qslot = qslot;
  P.out = out; P.lse = lse;
  P.err = err;
  P.part = part;
  const int64_t d = geom->head_dim;
  P.kv_layer_off = int64_t(layer) * geom->num_blocks * geom->num_kv_heads * geom->block_size * d;
  P.qwin_layer_off = int64_t(layer) * geom->max_slots * geom->num_q_heads * geom->window * d;
  P.qlse_layer_off = int64_t(layer) * geom->max_slots * geom->num_q_heads * geom->window;
  P.table_stride = table_stride; P.num_blocks = geom->num_blocks; P.b = geom->block_size;
  P.h_kv = geom->num_kv_heads; P.w = geom->window; P.max_slots = geom->max_slots;
  P.split_tokens = split_tokens; P.max_splits = max_splits; P.max_seq_len = max_seq_len;
  P.waves = waves;
  P.qk_scale = kLog2e / std::sqrt(float(d));
  P.log2b = __builtin_ctz(unsigned(geom->block_size));

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int g = group_size(geom);
  if (geom->dtype == ZP_DTYPE_BF16) {
    if (d == 128) dispatch_group<bf16_t, 128>(g, P, batch, s);
    else dispatch_group<bf16_t, 64>(g, P, batch, s);
  } else {
    if (d == 128) dispatch_group<float, 128>(g, P, batch, s);
    else dispatch_group<float, 64>(g, P, batch, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZP_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return ZP_OK;
}

// Library-owned split partials of zp_paged_decode_noalloc: one array per GPU
// (each device that loads the library holds its own copy until the process
// ends). Host code must not pass `scratch` itself to a kernel: its name is a
// host-side stand-in. The device address comes from hipGetSymbolAddress,
// taken once per device on that device's first call and kept here.
static __device__ __align__(256) unsigned char scratch[ZP_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static zp_status scratch_for_current_device(void** ptr, const char* who) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(ZP_EHIP, "%s: no current HIP device", who);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ZP_EHIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", who, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ZP_OK;
}

}  // namespace zp

using namespace zp;

extern "C" size_t zp_decode_workspace_size(const zp_geom* geom, int32_t batch,
                                           int32_t max_seq_len) {
  if (validate_geom(geom, "zp_decode_workspace_size") != ZP_OK || batch < 0 || max_seq_len < 0)
    return 0;
  return decode_ws_layout(geom, batch, max_seq_len, nullptr, nullptr, nullptr, nullptr);
}

extern "C" zp_status zp_paged_decode(const zp_geom* geom, const zp_cache* cache, int32_t layer,
                                     int32_t batch, const void* q, const void* k_new,
                                     const void* v_new, const int32_t* block_tables,
                                     int32_t table_stride, const int32_t* seq_lens,
                                     int32_t max_seq_len, const int32_t* qslot, void* out,
                                     float* lse, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  const char* who = "zp_paged_decode";
  size_t need = 0, p_off = 0;
  int32_t split_tokens = 0, max_splits = 0, waves = 0;
  zp_status st = decode_prepare(geom, cache, layer, batch, q, k_new, v_new, block_tables,
                                table_stride, seq_lens, max_seq_len, qslot, out, who, &need,
                                &p_off, &split_tokens, &max_splits, &waves);
  if (st != ZP_OK || batch == 0) return st;
  if (!workspace) return fail(ZP_EINVAL, "%s: NULL workspace", who);
  if (workspace_bytes < need)
    return fail(ZP_EINVAL, "%s: workspace %zu bytes, need %zu", who, workspace_bytes, need);
  char* ws = static_cast<char*>(workspace);
  return decode_enqueue(geom, cache, layer, batch, q, k_new, v_new, block_tables, table_stride,
                        seq_lens, max_seq_len, qslot, out, lse,
                        reinterpret_cast<float*>(ws + p_off), reinterpret_cast<uint32_t*>(ws),
                        split_tokens, max_splits, waves, stream, who);
}

extern "C" zp_status zp_paged_decode_noalloc(const zp_geom* geom, const zp_cache* cache,
                                             int32_t layer, int32_t batch, const void* q,
                                             const void* k_new, const void* v_new,
                                             const int32_t* block_tables, int32_t table_stride,
                                             const int32_t* seq_lens, int32_t max_seq_len,
                                             const int32_t* qslot, void* out, float* lse,
                                             uint32_t* errors, void* stream) {
  const char* who = "zp_paged_decode_noalloc";
  size_t need = 0, p_off = 0;
  int32_t split_tokens = 0, max_splits = 0, waves = 0;
  zp_status st = decode_prepare(geom, cache, layer, batch, q, k_new, v_new, block_tables,
                                table_stride, seq_lens, max_seq_len, qslot, out, who, &need,
                                &p_off, &split_tokens, &max_splits, &waves);
  if (st != ZP_OK || batch == 0) return st;
  // the partials need need - p_off bytes (the workspace header is not used:
  // error bits go to *errors)
  const size_t part_bytes = need - p_off;
  if (part_bytes > size_t(ZP_DECODE_SCRATCH_BYTES))
    return fail(ZP_EINVAL, "%s: this call needs %zu bytes of split partials, more than the "
                "%d-byte static scratch; use zp_paged_decode with a workspace", who, part_bytes,
                ZP_DECODE_SCRATCH_BYTES);
  void* base = nullptr;
  st = scratch_for_current_device(&base, who);
  if (st != ZP_OK) return st;
  return decode_enqueue(geom, cache, layer, batch, q, k_new, v_new, block_tables, table_stride,
                        seq_lens, max_seq_len, qslot, out, lse, static_cast<float*>(base), errors,
                        split_tokens, max_splits, waves, stream, who);
}
