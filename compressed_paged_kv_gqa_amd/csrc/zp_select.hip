// Top-k selection and in-order compaction of K, V and F (gfx950).
//
// Zipage (arXiv 2603.08743): Sec. 4.2 (keep the k = (N_max - 1) b entries with
// the highest scores; the window carries +inf), App. C.6 (top-k tag, then a
// two-pointer move that packs the kept entries densely and in order; the
// global-score cache F moves with K and V, one element per token instead of
// d), Sec. 4.4 (the packed entries go to target blocks, fresh ones for shared
// prefix blocks).
//
// Two launches:
//  1. Selection, one workgroup per (kv-head, request, layer): radix select
//     over order-preserving 32-bit keys of the fp32 scores (4 passes of 8
//     bits, LDS histogram) finds the k-th largest key; ties at that key go
//     to the highest token indices; the kept list is written ascending.
//     Units of up to 8192 tokens (select_fast_kernel) hold their keys in
//     registers, 16 or 32 per thread, and settle ties and ranks with wave
//     ballots and one scanned table of per-(row, wave) counts; longer ones
//     (select_kernel) stream the scores per pass and use a selection bitmap
//     in LDS with block scans.
//  2. compact_kernel, one workgroup per (128-byte slice of a token row, K or
//     V, kv-head, request, layer), with the kept list and both block tables
//     staged in LDS: the kept rows' slices are moved in chunks: every thread
//     loads its rows, the workgroup waits until all loads of the chunk have
//     completed, then stores. Destination slot j <= source slot kept[j] and
//     targets are either the same block or a fresh one, so no chunk reads a
//     slot that an earlier chunk wrote, and no chunk writes a slot a later
//     chunk still has to read before that read has completed. Different
//     workgroups touch disjoint bytes. The global-score entries move with the
//     first slice of K.
#include "zp_device.h"
#include "zp_internal.h"

namespace zp {

constexpr int kKeepMax = 8192;
constexpr int kSelMaxTokens = 65536;

struct SelectParams {
  const float* scores;
  const float* f_new;  // updated global scores to move into F, or NULL
  void* kc;
  void* vc;
  float* gscore;
  const int32_t* src_tables;
  const int32_t* num_blocks;
  const int32_t* dst_tables;
  int32_t* kept_out;
  int32_t* status;   // [layer_count][nreq][h_kv]: 1 = selection done, move it
  int32_t* kept_ws;  // [layer_count][nreq][h_kv][keep] ascending kept indices
  uint32_t* err;
  int64_t scores_stride;
  int64_t kv_layer_elems, f_layer_elems;
  int32_t src_stride, dst_stride;
  int32_t layer_begin, nreq, h_kv, b, num_blocks_total, max_blocks, keep;
  uint32_t flags;
};

// Order-preserving map of a float to uint32 (larger float -> larger key).
// -0 is folded onto +0 and NaN onto the smallest key.
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;
  if (f == 0.f) f = 0.f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 256 threads of the workgroup.
__device__ int block_inclusive_scan(int v, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  __syncthreads();
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
  for (int i = 0; i < wv; ++i) v += wsum[i];
  return v;
}

// Shared start of both selection kernels: clears the unit's status, checks
// its length and keep, and validates every block id the move will touch
// before anything is touched. Returns n (the unit's token count), or -1 when
// the unit must be skipped (errors flagged). Workgroup-uniform.
__device__ int select_prologue(const SelectParams& P, int z, int h, int r, int* sh_bad) {
  const int tid = threadIdx.x;
  const int N = P.num_blocks[r];
  int32_t* status = P.status + (int64_t)z * P.h_kv + h;
  if (tid == 0) *status = 0;  // nothing to move unless the selection completes
  if (N <= 0) return -1;
  if (N > P.max_blocks || N > P.src_stride) {
    if (tid == 0) flag_error(P.err, ZP_DEVERR_SEQ_LEN);
    return -1;
  }
  const int n = N * P.b;
  if (P.keep > n) {
    if (tid == 0) flag_error(P.err, ZP_DEVERR_KEEP);
    return -1;
  }
  const int32_t* stab = P.src_tables + (int64_t)r * P.src_stride;
  const int32_t* dtab = P.dst_tables + (int64_t)r * P.dst_stride;
  const bool compact = !(P.flags & ZP_SELECT_NO_COMPACT);
  if (tid == 0) *sh_bad = 0;
  __syncthreads();
  for (int i = tid; i < N; i += blockDim.x) {
    const int pg = stab[i];
    if (pg < 0 || pg >= P.num_blocks_total) *sh_bad = 1;
  }
  if (compact)
    for (int i = tid; i < (P.keep + P.b - 1) / P.b; i += blockDim.x) {
      const int pg = dtab[i];
      if (pg < 0 || pg >= P.num_blocks_total) *sh_bad = 1;
    }
  __syncthreads();
  if (*sh_bad) {
    if (tid == 0) flag_error(P.err, ZP_DEVERR_BLOCK_ID);
    return -1;
  }
  return n;
}

// The bin of the current radix digit that holds the krem-th largest key:
// thread tid takes bin 255 - tid, and a block scan gives the count of keys
// in higher bins (`above`). The selected bin is the one with above < krem
// <= above + its count (the first bin from the top when krem = 0). Updates
// prefix / krem in every thread.
__device__ __forceinline__ void radix_pick(const uint32_t* hist, int shift, int* wsum,
                                           uint32_t* sh_prefix, uint32_t* sh_krem,
                                           uint32_t& prefix, uint32_t& krem) {
  const int tid = threadIdx.x;
  const int v = 255 - tid;
  const int hv = (int)hist[v];
  const int incl = block_inclusive_scan(hv, wsum);
  const uint32_t above = (uint32_t)(incl - hv);
  if (krem == 0 ? tid == 0 : (above < krem && krem <= (uint32_t)incl)) {
    *sh_prefix = prefix | (uint32_t(v) << shift);
    *sh_krem = krem - above;
  }
  __syncthreads();
  prefix = *sh_prefix;
  krem = *sh_krem;
  __syncthreads();
}

__global__ __launch_bounds__(256) void select_kernel(SelectParams P) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t bitmap[kSelMaxTokens / 32];
  __shared__ int32_t kept[kKeepMax];
  __shared__ int wsum[4];
  __shared__ uint32_t sh_prefix, sh_krem;
  __shared__ int sh_bad;

  const int h = blockIdx.x, r = blockIdx.y, li = blockIdx.z;
  const int z = li * P.nreq + r;
  const int tid = threadIdx.x;
  const int n = select_prologue(P, z, h, r, &sh_bad);
  if (n < 0) return;
  const int keep = P.keep;
  const bool compact = !(P.flags & ZP_SELECT_NO_COMPACT);
  int32_t* status = P.status + (int64_t)z * P.h_kv + h;

  const float* sc = P.scores + ((int64_t)z * P.h_kv + h) * P.scores_stride;

  // 1. Radix select of the keep-th largest key.
  uint32_t prefix = 0, pmask = 0, krem = keep;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int t = tid; t < n; t += 256) {
      const uint32_t k = order_key(sc[t]);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    radix_pick(hist, shift, wsum, &sh_prefix, &sh_krem, prefix, krem);
    pmask |= 255u << shift;
  }
  const uint32_t thr = prefix;  // key of the keep-th largest score
  // krem = how many of the keys equal to thr are kept (the highest indices).

  // 2. Selection bitmap; equal keys counted from the end. Chunks of 1024
  // keys, 4 consecutive ones per thread, from the last chunk to the first;
  // within a chunk thread tid takes group 255 - tid, so an inclusive scan
  // over the threads counts the equal keys at higher indices. Each chunk's
  // scores are loaded one chunk ahead, so their latency overlaps the scan
  // of the chunk before.
  constexpr int GRP = 4, CH = 256 * GRP;
  const int nchunks = (n + CH - 1) / CH;
  int carry = 0;  // equal keys already seen in later chunks
  float s_next[GRP];
  auto load_group = [&](int c, float (&s)[GRP]) __attribute__((always_inline)) {
    const int t0 = c * CH + GRP * (255 - tid);
#pragma unroll
    for (int g = 0; g < GRP; ++g) s[g] = t0 + g < n ? sc[t0 + g] : 0.f;
  };
  load_group(nchunks - 1, s_next);
  for (int c = nchunks - 1; c >= 0; --c) {
    const int t0 = c * CH + GRP * (255 - tid);
    float s_cur[GRP];
#pragma unroll
    for (int g = 0; g < GRP; ++g) s_cur[g] = s_next[g];
    if (c > 0) load_group(c - 1, s_next);
    uint32_t k[GRP];
    uint32_t eqm = 0;
    int cnt = 0;
#pragma unroll
    for (int g = 0; g < GRP; ++g) {
      const bool valid = t0 + g < n;
      k[g] = valid ? order_key(s_cur[g]) : 0u;
      const bool e = valid && k[g] == thr;
      eqm |= uint32_t(e) << g;
      cnt += e;
    }
    const int incl = block_inclusive_scan(cnt, wsum);
    int later = carry + incl - cnt;  // equal keys above this group
    uint32_t selm = 0;
#pragma unroll
    for (int g = GRP - 1; g >= 0; --g) {  // highest index of the group first
      const bool e = (eqm >> g) & 1u;
      if (t0 + g < n && (k[g] > thr || (e && later < (int)krem))) selm |= 1u << g;
      later += e;
    }
    if (t0 < n) {
      const int w = t0 >> 5, sh = t0 & 31;
      atomicAnd(&bitmap[w], ~(((1u << GRP) - 1u) << sh));
      atomicOr(&bitmap[w], selm << sh);
    }
    __syncthreads();
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }

  // 3. Ascending kept list, 4 consecutive indices per thread.
  int base = 0;
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * CH + GRP * tid;
    const uint32_t selm = t0 < n ? (bitmap[t0 >> 5] >> (t0 & 31)) & ((1u << GRP) - 1u) : 0u;
    const int cnt = __popc(selm);
    const int incl = block_inclusive_scan(cnt, wsum);
    int pos = base + incl - cnt;
#pragma unroll
    for (int g = 0; g < GRP; ++g) {
      if ((selm >> g) & 1u) {
        if (pos < keep) kept[pos] = t0 + g;
        ++pos;
      }
    }
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  __syncthreads();
  int32_t* kw = P.kept_ws + ((int64_t)z * P.h_kv + h) * keep;
  for (int j = tid; j < keep; j += 256) kw[j] = kept[j];
  if (P.kept_out) {
    int32_t* ko = P.kept_out + ((int64_t)z * P.h_kv + h) * keep;
    for (int j = tid; j < keep; j += 256) ko[j] = kept[j];
  }
  if (tid == 0 && compact) *status = 1;
}

// Selection for units of at most NT KPT tokens, keys held in registers:
// thread tid of the NT holds tokens tid + NT i (i < KPT), so index order is
// (i, wave, lane). The radix passes are those of select_kernel; in the first
// one a wave's lanes hold neighbouring tokens, whose keys mostly share the
// top byte, so each lane group with the same bin adds its count once. The
// tie rule (equal keys at the threshold go to the highest indices) and the
// ascending kept list come from per-row wave ballots and a table of
// per-(row, wave) counts that one wavefront scans (suffix sums for the ties,
// prefix sums for the ranks). Same output as select_kernel.
template <int NT>
__device__ __forceinline__ int block_incl_scan_n(int v, int* wsum) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  __syncthreads();
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i)
    if (i < wv) v += wsum[i];
  return v;
}

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void select_fast_kernel(SelectParams P) {
  constexpr int NW = NT / 64;
  constexpr int NE = NW * KPT;           // (row, wave) entries, in index order
  constexpr int EPL = (NE + 63) / 64;    // entries per lane of the scanning wavefront
  __shared__ uint32_t hist[256];
  __shared__ int wsum[NW];
  __shared__ uint32_t sh_prefix, sh_krem;
  __shared__ int sh_bad;
  __shared__ int cnt[EPL * 64], scn[EPL * 64];

  const int h = blockIdx.x, r = blockIdx.y, li = blockIdx.z;
  const int z = li * P.nreq + r;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int keep = P.keep;
  const bool compact = !(P.flags & ZP_SELECT_NO_COMPACT);
  const float* sc = P.scores + ((int64_t)z * P.h_kv + h) * P.scores_stride;
  // The scores are requested before the block ids are checked, so the two
  // round trips overlap (n is not known yet: max_blocks bounds the reads,
  // which scores_stride covers).
  const int n_cap = P.max_blocks * P.b;
  float sv[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) sv[i] = tid + NT * i < n_cap ? sc[tid + NT * i] : 0.f;
  const int n = select_prologue(P, z, h, r, &sh_bad);
  if (n < 0) return;

  uint32_t key[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] = tid + NT * i < n ? order_key(sv[i]) : 0u;
  // 1. Radix select of the keep-th largest key.
  uint32_t prefix = 0, pmask = 0, krem = keep;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    if (pass == 0) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool in = tid + NT * i < n;
        const uint32_t bin = key[i] >> 24;
        const uint32_t lead = __builtin_amdgcn_readfirstlane(in ? bin : 256u);
        const uint64_t same = __ballot(in && bin == lead);
        if (same != 0 && lane == (int)__builtin_ctzll(same)) atomicAdd(&hist[lead], (uint32_t)__popcll(same));
        if (in && bin != lead) atomicAdd(&hist[bin], 1u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        if (tid + NT * i < n && (key[i] & pmask) == prefix)
          atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    {  // the bin holding the krem-th largest key, from the top (see radix_pick)
      const int v = 255 - tid;
      const int hv = tid < 256 ? (int)hist[v] : 0;
      const int incl = block_incl_scan_n<NT>(hv, wsum);
      const uint32_t above = (uint32_t)(incl - hv);
      if (tid < 256 && (krem == 0 ? tid == 0 : (above < krem && krem <= (uint32_t)incl))) {
        sh_prefix = prefix | (uint32_t(v) << shift);
        sh_krem = krem - above;
      }
      __syncthreads();
      prefix = sh_prefix;
      krem = sh_krem;
      __syncthreads();
    }
    pmask |= 255u << shift;
  }
  const uint32_t thr = prefix;

  const uint64_t below = (1ull << lane) - 1ull;  // lanes under this one
  const uint64_t above = ~below << 1;            // lanes over this one
  // 2. Ties: keys equal to thr at higher indices, from per-(row, wave) counts
  // summed from the end of the index order.
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const uint64_t m = __ballot(tid + NT * i < n && key[i] == thr);
    if (lane == 0) cnt[i * NW + wv] = __popcll(m);
  }
  __syncthreads();
  if (wv == 0) {  // scn[e] = sum of cnt over entries after e
    int c[EPL], tot = 0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      c[k] = lane * EPL + k < NE ? cnt[lane * EPL + k] : 0;
      tot += c[k];
    }
    int suf = tot;  // inclusive suffix over lanes >= this one
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_down(suf, d, 64);
      if (lane + d < 64) suf += o;
    }
    int after = suf - tot;
#pragma unroll
    for (int k = EPL - 1; k >= 0; --k) { scn[lane * EPL + k] = after; after += c[k]; }
  }
  __syncthreads();
  uint32_t selm = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool valid = tid + NT * i < n;
    const bool eq = valid && key[i] == thr;
    const uint64_t m = __ballot(eq);
    const uint32_t later = (uint32_t)scn[i * NW + wv] + (uint32_t)__popcll(m & above);
    if (valid && (key[i] > thr || (eq && later < krem))) selm |= 1u << i;
  }
  __syncthreads();  // scn is reused below
  // 3. Ranks in index order: per-(row, wave) counts of selected keys,
  // exclusive prefix sums over the entries, then the lanes below.
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const uint64_t m = __ballot((selm >> i) & 1u);
    if (lane == 0) cnt[i * NW + wv] = __popcll(m);
  }
  __syncthreads();
  if (wv == 0) {
    int c[EPL], tot = 0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      c[k] = lane * EPL + k < NE ? cnt[lane * EPL + k] : 0;
      tot += c[k];
    }
    int pre = tot;  // inclusive prefix over lanes <= this one
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(pre, d, 64);
      if (lane >= d) pre += o;
    }
    int before = pre - tot;
#pragma unroll
    for (int k = 0; k < EPL; ++k) { scn[lane * EPL + k] = before; before += c[k]; }
    // exactly keep keys are selected by construction; should that ever
    // fail, nothing is moved and the error bit is set
    if (lane == 63) sh_bad = (before != keep);
  }
  __syncthreads();
  if (sh_bad) {
    if (tid == 0) flag_error(P.err, ZP_DEVERR_KEEP);
    return;
  }
  int32_t* kw = P.kept_ws + ((int64_t)z * P.h_kv + h) * keep;
  int32_t* ko = P.kept_out ? P.kept_out + ((int64_t)z * P.h_kv + h) * keep : nullptr;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool sl = (selm >> i) & 1u;
    const uint64_t m = __ballot(sl);
    const int pos = scn[i * NW + wv] + __popcll(m & below);
    if (sl && pos < keep) {
      kw[pos] = tid + NT * i;
      if (ko) ko[pos] = tid + NT * i;
    }
  }
  if (tid == 0 && compact) P.status[(int64_t)z * P.h_kv + h] = 1;
}

// Moves the kept rows of one (layer, request, kv-head): this workgroup takes
// byte slice `sl` (128 bytes = 8 lanes x 16 B) of every row of K (kv = 0) or
// V (kv = 1), in chunks of 256 rows: every thread loads its rows, the
// workgroup waits until all loads of the chunk have completed, then stores.
// Destination slot j <= source slot kept[j] and targets are either the same
// block or a fresh one, so no chunk reads a slot that an earlier chunk wrote,
// and no chunk writes a slot a later chunk still has to read before that
// read has completed. The global-score entries (one per row, one row per
// thread) move with the first slice of K.
template <typename T, int D>
__global__ __launch_bounds__(256) void compact_kernel(SelectParams P) {
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int SLICES = ROWB / 128;
  constexpr int RPP = 256 / 8;           // rows per pass
  constexpr int PASSES = 8;
  constexpr int CHUNK = RPP * PASSES;    // rows per chunk (256, one per thread for F)
  // LDS: the kept list, then the request's source and target block ids, so
  // a row's address takes LDS reads only and the row loads never wait on a
  // block-id load (the memory counter is in order: waiting for one load
  // waits for every row load issued before it).
  extern __shared__ int32_t kept[];      // [keep] [max_blocks] [ceil(keep / b)]

  const int sl = blockIdx.x % SLICES, kv = blockIdx.x / SLICES;
  const int h = blockIdx.y, z = blockIdx.z;
  const int r = z % P.nreq;
  const int layer = P.layer_begin + z / P.nreq;
  const int tid = threadIdx.x;
  if (P.status[(int64_t)z * P.h_kv + h] != 1) return;  // selection flagged an error
  const int keep = P.keep;
  const int b = P.b;
  const int lb = __builtin_ctz((unsigned)b);  // b is a power of two
  const int N = P.num_blocks[r];              // <= max_blocks: the selection checked it
  const int nd = (keep + b - 1) / b;
  int32_t* stab = kept + keep;
  int32_t* dtab = stab + P.max_blocks;
  const int32_t* kw = P.kept_ws + ((int64_t)z * P.h_kv + h) * keep;
  for (int j = tid; j < keep; j += 256) kept[j] = kw[j];
  for (int j = tid; j < N; j += 256) stab[j] = P.src_tables[(int64_t)r * P.src_stride + j];
  for (int j = tid; j < nd; j += 256) dtab[j] = P.dst_tables[(int64_t)r * P.dst_stride + j];
  __syncthreads();
  char* base = reinterpret_cast<char*>(kv ? P.vc : P.kc) + layer * P.kv_layer_elems * (int64_t)sizeof(T);
  float* fc = (P.gscore && kv == 0 && sl == 0) ? P.gscore + layer * P.f_layer_elems : nullptr;
  const float* fnew = P.f_new ? P.f_new + ((int64_t)z * P.h_kv + h) * P.scores_stride : nullptr;
  const int64_t page_bytes = (int64_t)P.h_kv * b * ROWB;
  const int64_t head_bytes = (int64_t)h * b * ROWB;
  const int rr = tid / 8;
  const int lane_off = sl * 128 + (tid % 8) * 16;
  for (int j0 = 0; j0 < keep; j0 += CHUNK) {
    uint4 v[PASSES];
    float fv = 0.f;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int j = j0 + ps * RPP + rr;
      if (j < keep) {
        const int t = kept[j];
        v[ps] = ld16(base + (int64_t)stab[t >> lb] * page_bytes + head_bytes +
                     (int64_t)(t & (b - 1)) * ROWB + lane_off);
      }
    }
    if (fc && j0 + tid < keep) {
      const int t = kept[j0 + tid];
      fv = fnew ? fnew[t] : fc[((int64_t)stab[t >> lb] * P.h_kv + h) * b + (t & (b - 1))];
    }
    __builtin_amdgcn_s_waitcnt(0);  // every load of the chunk has returned
    __syncthreads();
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int j = j0 + ps * RPP + rr;
      if (j < keep)
        st16(base + (int64_t)dtab[j >> lb] * page_bytes + head_bytes + (int64_t)(j & (b - 1)) * ROWB +
                 lane_off, v[ps]);
    }
    if (fc && j0 + tid < keep) {
      const int j = j0 + tid;
      fc[((int64_t)dtab[j >> lb] * P.h_kv + h) * b + (j & (b - 1))] = fv;
    }
  }
}

template <typename T, int D>
static void launch_select(const SelectParams& P, int layer_count, hipStream_t s) {
  const dim3 gs(P.h_kv, P.nreq, layer_count);
  const int64_t n_max = int64_t(P.max_blocks) * P.b;
  constexpr int NT = 256;  // 1024 threads of 4 or 8 keys each measured slower
  if (n_max <= 4096)
    hipLaunchKernelGGL((select_fast_kernel<NT, 4096 / NT>), gs, dim3(NT), 0, s, P);
  else if (n_max <= 8192)
    hipLaunchKernelGGL((select_fast_kernel<NT, 8192 / NT>), gs, dim3(NT), 0, s, P);
  else
    hipLaunchKernelGGL(select_kernel, gs, dim3(256), 0, s, P);
  if (!(P.flags & ZP_SELECT_NO_COMPACT)) {
    constexpr int SLICES = D * (int)sizeof(T) / 128;
    const size_t lds = sizeof(int32_t) * (size_t(P.keep) + P.max_blocks + (P.keep + P.b - 1) / P.b);
    hipLaunchKernelGGL((compact_kernel<T, D>), dim3(2 * SLICES, P.h_kv, P.nreq * layer_count),
                       dim3(256), lds, s, P);
  }
}

}  // namespace zp

using namespace zp;

static size_t select_ws_layout(const zp_geom* g, int32_t layer_count, int32_t nreq, int32_t keep,
                               size_t* status_off, size_t* kept_off) {
  const size_t items = size_t(layer_count) * nreq * g->num_kv_heads;
  const size_t so = kWsHeader;
  const size_t ko = round_up(so + items * sizeof(int32_t), 256);
  if (status_off) *status_off = so;
  if (kept_off) *kept_off = ko;
  return round_up(ko + items * size_t(keep) * sizeof(int32_t), 256);
}

extern "C" size_t zp_select_workspace_size(const zp_geom* geom, int32_t layer_count,
                                           int32_t nreq, int32_t keep) {
  if (validate_geom(geom, "zp_select_workspace_size") != ZP_OK || layer_count < 0 || nreq < 0 ||
      keep < 0)
    return 0;
  return select_ws_layout(geom, layer_count, nreq, keep, nullptr, nullptr);
}

extern "C" zp_status zp_select_compact(const zp_geom* geom, const zp_cache* cache,
                                       int32_t layer_begin, int32_t layer_count, int32_t nreq,
                                       const float* scores, const float* f_new,
                                       int64_t scores_stride,
                                       const int32_t* src_tables, int32_t src_stride,
                                       const int32_t* num_blocks, int32_t max_blocks,
                                       const int32_t* dst_tables, int32_t dst_stride,
                                       int32_t keep, int32_t* kept_idx, uint32_t flags,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  zp_status st = validate_geom(geom, "zp_select_compact");
  if (st != ZP_OK) return st;
  if (!cache || !cache->k || !cache->v) return fail(ZP_EINVAL, "zp_select_compact: cache NULL");
  if (layer_begin < 0 || layer_count < 0 || layer_begin + layer_count > geom->num_layers)
    return fail(ZP_EINVAL, "zp_select_compact: layer range outside the cache");
  if (nreq < 0 || max_blocks < 0 || src_stride <= 0)
    return fail(ZP_EINVAL, "zp_select_compact: bad nreq/max_blocks/src_stride");
  if (flags & ~uint32_t(ZP_SELECT_NO_COMPACT))
    return fail(ZP_EINVAL, "zp_select_compact: unknown flags 0x%x", flags);
  if (keep < 1 || keep > kKeepMax)
    return fail(ZP_EINVAL, "zp_select_compact: keep %d outside [1, %d]", keep, kKeepMax);
  if (int64_t(max_blocks) * geom->block_size > kSelMaxTokens)
    return fail(ZP_EINVAL, "zp_select_compact: max_blocks*b above %d tokens", kSelMaxTokens);
  const bool compact = !(flags & ZP_SELECT_NO_COMPACT);
  if (compact && (!dst_tables || dst_stride <= 0 || int64_t(dst_stride) * geom->block_size < keep))
    return fail(ZP_EINVAL, "zp_select_compact: dst_tables must hold keep tokens");
  if (nreq == 0 || layer_count == 0 || max_blocks == 0) return ZP_OK;
  if (!scores || !src_tables || !num_blocks || !workspace)
    return fail(ZP_EINVAL, "zp_select_compact: NULL buffer");
  if (scores_stride < int64_t(max_blocks) * geom->block_size)
    return fail(ZP_EINVAL, "zp_select_compact: scores_stride < max_blocks*b");
  size_t status_off, kept_off;
  const size_t need = select_ws_layout(geom, layer_count, nreq, keep, &status_off, &kept_off);
  if (workspace_bytes < need)
    return fail(ZP_EINVAL, "zp_select_compact: workspace %zu bytes, need %zu", workspace_bytes, need);
  if (nreq > 65535 || layer_count > 65535)
    return fail(ZP_EINVAL, "zp_select_compact: nreq and layer_count must be <= 65535");

  SelectParams P{};
  P.scores = scores; P.f_new = f_new; P.scores_stride = scores_stride;
  P.kc = cache->k; P.vc = cache->v; P.gscore = cache->gscore;
  P.src_tables = src_tables; P.src_stride = src_stride; P.num_blocks = num_blocks;
  P.dst_tables = dst_tables ? dst_tables : src_tables;
  P.dst_stride = dst_tables ? dst_stride : src_stride;
  P.kept_out = kept_idx;
  P.err = static_cast<uint32_t*>(workspace);
  P.status = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + status_off);
  P.kept_ws = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + kept_off);
  const int64_t d = geom->head_dim;
  P.kv_layer_elems = int64_t(geom->num_blocks) * geom->num_kv_heads * geom->block_size * d;
  P.f_layer_elems = int64_t(geom->num_blocks) * geom->num_kv_heads * geom->block_size;
  P.layer_begin = layer_begin; P.nreq = nreq; P.h_kv = geom->num_kv_heads;
  P.b = geom->block_size; P.num_blocks_total = geom->num_blocks; P.max_blocks = max_blocks;
  P.keep = keep; P.flags = flags;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (geom->dtype == ZP_DTYPE_BF16) {
    if (d == 128) launch_select<bf16_t, 128>(P, layer_count, s);
    else launch_select<bf16_t, 64>(P, layer_count, s);
  } else {
    if (d == 128) launch_select<float, 128>(P, layer_count, s);
    else launch_select<float, 64>(P, layer_count, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZP_EHIP, "zp_select_compact: launch failed: %s", hipGetErrorString(e));
  return ZP_OK;
}

extern "C" zp_status zp_workspace_errors(const void* workspace, uint32_t* flags, void* stream) {
  if (!workspace || !flags) return fail(ZP_EINVAL, "zp_workspace_errors: NULL argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(ZP_EHIP, "zp_workspace_errors: %s", hipGetErrorString(e));
  return ZP_OK;
}

namespace zp {
__global__ void clear_word_kernel(uint32_t* p) { *p = 0u; }
}  // namespace zp

extern "C" zp_status zp_workspace_clear_errors(void* workspace, void* stream) {
  if (!workspace) return fail(ZP_EINVAL, "zp_workspace_clear_errors: NULL workspace");
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(workspace));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZP_EHIP, "zp_workspace_clear_errors: %s", hipGetErrorString(e));
  return ZP_OK;
}
