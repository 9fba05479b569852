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
//  1. select_kernel, one workgroup per (kv-head, request, layer): radix
//     select over order-preserving 32-bit keys of the fp32 scores (4 passes
//     of 8 bits, LDS histogram) finds the k-th largest key; ties at that key
//     go to the highest token indices (a backward block scan, 4 keys per
//     thread), giving a selection bitmap in LDS; a forward block scan turns
//     it into the ascending kept list, written to the workspace (and to
//     kept_idx). The bin holding the k-th key is found with a block scan
//     over the 256 bins.
//  2. compact_kernel, one workgroup per (128-byte slice of a token row, K or
//     V, kv-head, request, layer): the kept rows' slices are moved in chunks:
//     every thread loads its rows, the workgroup waits until all loads of the
//     chunk have completed, then stores. Destination slot j <= source slot
//     kept[j] and targets are either the same block or a fresh one, so no
//     chunk reads a slot that an earlier chunk wrote, and no chunk writes a
//     slot a later chunk still has to read before that read has completed.
//     Different workgroups touch disjoint bytes. The global-score entries
//     move with the first slice of K.
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
  const int N = P.num_blocks[r];
  int32_t* status = P.status + (int64_t)z * P.h_kv + h;
  if (tid == 0) *status = 0;  // nothing to move unless the selection completes
  if (N <= 0) return;
  if (N > P.max_blocks || N > P.src_stride) {
    if (tid == 0) flag_error(P.err, ZP_DEVERR_SEQ_LEN);
    return;
  }
  const int n = N * P.b;
  const int keep = P.keep;
  if (keep > n) {
    if (tid == 0) flag_error(P.err, ZP_DEVERR_KEEP);
    return;
  }
  const int32_t* stab = P.src_tables + (int64_t)r * P.src_stride;
  const int32_t* dtab = P.dst_tables + (int64_t)r * P.dst_stride;
  const bool compact = !(P.flags & ZP_SELECT_NO_COMPACT);
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  // Validate every block id the move will touch before touching anything.
  for (int i = tid; i < N; i += 256) {
    const int pg = stab[i];
    if (pg < 0 || pg >= P.num_blocks_total) sh_bad = 1;
  }
  if (compact)
    for (int i = tid; i < (keep + P.b - 1) / P.b; i += 256) {
      const int pg = dtab[i];
      if (pg < 0 || pg >= P.num_blocks_total) sh_bad = 1;
    }
  __syncthreads();
  if (sh_bad) {
    if (tid == 0) flag_error(P.err, ZP_DEVERR_BLOCK_ID);
    return;
  }

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
    // The bin holding the krem-th largest key: thread tid takes bin 255 - tid,
    // and a block scan gives the count of keys in higher bins (`above`). The
    // selected bin is the one with above < krem <= above + its count (the
    // first bin from the top when krem = 0).
    {
      const int v = 255 - tid;
      const int hv = (int)hist[v];
      const int incl = block_inclusive_scan(hv, wsum);
      const uint32_t above = (uint32_t)(incl - hv);
      if (krem == 0 ? tid == 0 : (above < krem && krem <= (uint32_t)incl)) {
        sh_prefix = prefix | (uint32_t(v) << shift);
        sh_krem = krem - above;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    krem = sh_krem;
    pmask |= 255u << shift;
    __syncthreads();
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


// Moves the kept rows of one (layer, request, kv-head): this workgroup takes
// byte slice `sl` (128 bytes = 8 lanes x 16 B) of every row of K (kv = 0) or
// V (kv = 1).
template <typename T, int D>
__global__ __launch_bounds__(256) void compact_kernel(SelectParams P) {
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int SLICES = ROWB / 128;
  constexpr int RPP = 256 / 8;           // rows per pass
  constexpr int PASSES = 8;
  constexpr int CHUNK = RPP * PASSES;    // rows per chunk (256)
  extern __shared__ int32_t kept[];      // [keep]

  const int sl = blockIdx.x % SLICES, kv = blockIdx.x / SLICES;
  const int h = blockIdx.y, z = blockIdx.z;
  const int r = z % P.nreq;
  const int layer = P.layer_begin + z / P.nreq;
  const int tid = threadIdx.x;
  if (P.status[(int64_t)z * P.h_kv + h] != 1) return;  // selection flagged an error
  const int keep = P.keep;
  const int b = P.b;
  const int32_t* kw = P.kept_ws + ((int64_t)z * P.h_kv + h) * keep;
  for (int j = tid; j < keep; j += 256) kept[j] = kw[j];
  __syncthreads();
  const int32_t* stab = P.src_tables + (int64_t)r * P.src_stride;
  const int32_t* dtab = P.dst_tables + (int64_t)r * P.dst_stride;
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
        v[ps] = ld16(base + (int64_t)stab[t / b] * page_bytes + head_bytes +
                     (int64_t)(t % b) * ROWB + lane_off);
      }
    }
    if (fc && j0 + tid < keep) {
      const int t = kept[j0 + tid];
      fv = fnew ? fnew[t] : fc[((int64_t)stab[t / b] * P.h_kv + h) * b + (t % b)];
    }
    __builtin_amdgcn_s_waitcnt(0);  // every load of the chunk has returned
    __syncthreads();
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int j = j0 + ps * RPP + rr;
      if (j < keep)
        st16(base + (int64_t)dtab[j / b] * page_bytes + head_bytes + (int64_t)(j % b) * ROWB +
                 lane_off, v[ps]);
    }
    if (fc && j0 + tid < keep) {
      const int j = j0 + tid;
      fc[((int64_t)dtab[j / b] * P.h_kv + h) * b + (j % b)] = fv;
    }
  }
}

template <typename T, int D>
static void launch_select(const SelectParams& P, int layer_count, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(P.h_kv, P.nreq, layer_count), dim3(256), 0, s, P);
  if (!(P.flags & ZP_SELECT_NO_COMPACT)) {
    constexpr int SLICES = D * (int)sizeof(T) / 128;
    hipLaunchKernelGGL((compact_kernel<T, D>), dim3(2 * SLICES, P.h_kv, P.nreq * layer_count),
                       dim3(256), sizeof(int32_t) * P.keep, s, P);
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
