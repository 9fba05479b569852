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
//  * q.k partial dot products are all-reduced inside each row group with DPP
//    (no LDS), softmax is online in exp2 form per chunk of tokens;
//  * the split partials (max, sum, unnormalised output) are merged by the
//    last workgroup of each (sequence, kv-head) to finish (device-scope
//    fence + counter), so one launch covers the whole step;
//  * the token being decoded is taken from k_new / v_new directly by the
//    split that covers it, which also writes it to its page: no other
//    workgroup reads that slot, so append and attention need no extra launch.
#include <cmath>

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
  const int32_t* tables;
  const int32_t* seq_lens;
  const int32_t* qslot;
  void* out;
  float* lse;
  float* part;        // [batch][h_kv][max_splits][G][D + 2]
  int32_t* counters;  // [batch][h_kv]
  uint32_t* err;
  int64_t kv_layer_off;    // element offset of the layer in K / V
  int64_t qwin_layer_off;  // element offset of the layer in Qwin
  int32_t table_stride, num_blocks, b, h_kv, w, max_slots;
  int32_t split_tokens, max_splits, max_seq_len;
  float qk_scale;  // log2(e) / sqrt(d)
};

template <typename T, int D, int G>
struct DecodeCfg {
  static constexpr int EPL = Vec16<T>::N;  // elements per lane per 16-byte load
  static constexpr int LPR = D / EPL;      // lanes per token row
  static constexpr int RPW = 64 / LPR;     // token rows per wavefront load
  static constexpr int U = 4;              // row loads in flight per lane (K and V each)
  static constexpr int TILE = RPW * U;     // tokens per wavefront iteration
  static constexpr int WAVES = 4;
};

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void paged_decode_kernel(DecodeParams P) {
  using C = DecodeCfg<T, D, G>;
  constexpr int EPL = C::EPL, LPR = C::LPR, RPW = C::RPW, U = C::U, TILE = C::TILE;
  constexpr int WAVES = C::WAVES;

  __shared__ float sm_m[WAVES][G];
  __shared__ float sm_l[WAVES][G];
  __shared__ float sm_o[WAVES][G][D];
  __shared__ int sm_last;

  const int split = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int n = P.seq_lens[seq];
  if (n <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int h_q = P.h_kv * G;
  const int64_t out_row = (int64_t)seq * h_q + (int64_t)kvh * G;  // first head of the group

  if (n > P.max_seq_len || n > (int64_t)P.table_stride * P.b) {
    // The launch does not cover this row: report, poison its outputs.
    if (split == 0) {
      if (tid == 0) flag_error(P.err, ZP_DEVERR_SEQ_LEN);
      T* out = reinterpret_cast<T*>(P.out);
      for (int i = tid; i < G * D; i += 256) out[out_row * D + i] = from_f32<T>(NAN);
      if (P.lse && tid < G) P.lse[out_row + tid] = NAN;
    }
    return;
  }
  const int nsplit = (n + P.split_tokens - 1) / P.split_tokens;
  if (split >= nsplit) return;
  const int t0 = split * P.split_tokens;
  const int t1 = min(n, t0 + P.split_tokens);
  const int row = lane / LPR;
  const int sub = lane % LPR;
  const int32_t* tab = P.tables + (int64_t)seq * P.table_stride;
  const T* kc = reinterpret_cast<const T*>(P.kc) + P.kv_layer_off;
  const T* vc = reinterpret_cast<const T*>(P.vc) + P.kv_layer_off;
  const T* knew = reinterpret_cast<const T*>(P.k_new) + ((int64_t)seq * P.h_kv + kvh) * D + sub * EPL;
  const T* vnew = reinterpret_cast<const T*>(P.v_new) + ((int64_t)seq * P.h_kv + kvh) * D + sub * EPL;
  const int64_t head_off = (int64_t)kvh * P.b * D + sub * EPL;  // within a page
  const int64_t page_elems = (int64_t)P.h_kv * P.b * D;

  // Query rows of the group, this lane's EPL dims, in fp32.
  float qf[G][EPL];
  {
    const T* qp = reinterpret_cast<const T*>(P.q) + out_row * D + sub * EPL;
#pragma unroll
    for (int h = 0; h < G; ++h) Vec16<T>::unpack(ld16(qp + (int64_t)h * D), qf[h]);
  }

  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
  }

  for (int base = t0 + wv * TILE; base < t1; base += WAVES * TILE) {
    uint4 kr[U], vr[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + u * RPW + row;
      valid[u] = t < t1;
      const int tt = valid[u] ? t : t0;
      const T* kp;
      const T* vp;
      if (tt == n - 1) {
        kp = knew;
        vp = vnew;
      } else {
        const int page = tab[tt / P.b];
        const bool ok = page >= 0 && page < P.num_blocks;
        if (!ok) {
          if (valid[u] && sub == 0) flag_error(P.err, ZP_DEVERR_BLOCK_ID);
          valid[u] = false;
        }
        const int64_t off = (ok ? page : 0) * page_elems + head_off + (int64_t)(tt % P.b) * D;
        kp = kc + off;
        vp = vc + off;
      }
      kr[u] = ld16(kp);
      vr[u] = ld16(vp);
    }

    // Logits, pre-multiplied by log2(e)/sqrt(d).
    float s[G][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[EPL];
      Vec16<T>::unpack(kr[u], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(qf[h][e], kf[e], acc);
        s[h][u] = acc;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float v = group_sum<LPR>(s[h][u]) * P.qk_scale;
        s[h][u] = valid[u] ? v : -INFINITY;
      }

    // Online softmax update per head over this chunk.
    float vf[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) Vec16<T>::unpack(vr[u], vf[u]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float cm = s[h][0];
#pragma unroll
      for (int u = 1; u < U; ++u) cm = fmaxf(cm, s[h][u]);
      cm = across_groups_max<LPR>(cm);
      const float mn = fmaxf(m[h], cm);
      if (mn == -INFINITY) continue;  // nothing visible yet
      const float alpha = exp2f(m[h] - mn);
      m[h] = mn;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = exp2f(s[h][u] - mn);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(p, vf[u][e], o[h][e]);
      }
    }

    // Append the decoded token to its page (only the split holding n-1).
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + u * RPW + row;
      if (t == n - 1 && t < t1) {
        const int page = tab[t / P.b];
        if (page >= 0 && page < P.num_blocks) {
          const int64_t off = (int64_t)page * page_elems + head_off + (int64_t)(t % P.b) * D;
          st16(const_cast<T*>(kc) + off, kr[u]);
          st16(const_cast<T*>(vc) + off, vr[u]);
        }
      }
    }
  }

  // Merge the row groups of the wavefront (m is already wavefront-uniform).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = across_groups_sum<LPR>(l[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = across_groups_sum<LPR>(o[h][e]);
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
        for (int i = tid; i < G * D; i += 256) {
          const int h = i / D, e = i % D;
          dst[(int64_t)h * P.w * D + e] = qp[i];
        }
      }
    }
  }

  // Combine the 4 wavefronts: each thread owns (head, dim) pairs.
  constexpr int PAIRS = G * D;
  float Mw[(PAIRS + 255) / 256], Lw[(PAIRS + 255) / 256], Ow[(PAIRS + 255) / 256];
#pragma unroll
  for (int k = 0; k < (PAIRS + 255) / 256; ++k) {
    const int i = tid + k * 256;
    Mw[k] = -INFINITY; Lw[k] = 0.f; Ow[k] = 0.f;
    if (i < PAIRS) {
      const int h = i / D, e = i % D;
      float M = sm_m[0][h];
#pragma unroll
      for (int w2 = 1; w2 < WAVES; ++w2) M = fmaxf(M, sm_m[w2][h]);
      float L = 0.f, O = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w2 = 0; w2 < WAVES; ++w2) {
          const float sc = exp2f(sm_m[w2][h] - M);
          L += sm_l[w2][h] * sc;
          O += sm_o[w2][h][e] * sc;
        }
      }
      Mw[k] = M; Lw[k] = L; Ow[k] = O;
    }
  }

  T* out = reinterpret_cast<T*>(P.out);
  if (nsplit == 1) {
#pragma unroll
    for (int k = 0; k < (PAIRS + 255) / 256; ++k) {
      const int i = tid + k * 256;
      if (i < PAIRS) {
        const int h = i / D, e = i % D;
        out[(out_row + h) * D + e] = from_f32<T>(Ow[k] / Lw[k]);
        if (P.lse && e == 0) P.lse[out_row + h] = (Mw[k] + log2f(Lw[k])) * kLn2;
      }
    }
    return;
  }

  // Several splits: publish this split's partial, the last one merges.
  const int64_t item = (int64_t)seq * P.h_kv + kvh;
  float* mypart = P.part + (item * P.max_splits + split) * G * (D + 2);
#pragma unroll
  for (int k = 0; k < (PAIRS + 255) / 256; ++k) {
    const int i = tid + k * 256;
    if (i < PAIRS) {
      const int h = i / D, e = i % D;
      mypart[h * (D + 2) + 2 + e] = Ow[k];
      if (e == 0) {
        mypart[h * (D + 2)] = Mw[k];
        mypart[h * (D + 2) + 1] = Lw[k];
      }
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int prev = atomicAdd(&P.counters[item], 1);
    sm_last = (prev == nsplit - 1);
  }
  __syncthreads();
  if (!sm_last) return;
  __threadfence();
  const float* parts = P.part + item * P.max_splits * G * (D + 2);
  for (int i = tid; i < PAIRS; i += 256) {
    const int h = i / D, e = i % D;
    float M = -INFINITY;
    for (int s2 = 0; s2 < nsplit; ++s2) M = fmaxf(M, parts[(s2 * G + h) * (D + 2)]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int s2 = 0; s2 < nsplit; ++s2) {
        const float* pp = parts + (s2 * G + h) * (D + 2);
        const float sc = exp2f(pp[0] - M);
        L += pp[1] * sc;
        O += pp[2 + e] * sc;
      }
    }
    out[(out_row + h) * D + e] = from_f32<T>(O / L);
    if (P.lse && e == 0) P.lse[out_row + h] = (M + log2f(L)) * kLn2;
  }
  if (tid == 0) P.counters[item] = 0;  // leave the workspace reusable
}

template <typename T, int D, int G>
static void launch_decode(const DecodeParams& P, int batch, hipStream_t stream) {
  dim3 grid(P.max_splits, P.h_kv, batch);
  hipLaunchKernelGGL((paged_decode_kernel<T, D, G>), grid, dim3(256), 0, stream, P);
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
                               size_t* counters_off, size_t* part_off, int32_t* split_tokens,
                               int32_t* max_splits) {
  const int32_t st = decode_split_tokens(g, batch, max_seq_len);
  const int32_t ms = std::max<int32_t>(1, (std::max<int32_t>(max_seq_len, 1) + st - 1) / st);
  const size_t items = size_t(batch) * g->num_kv_heads;
  const size_t c_off = kWsHeader;
  const size_t p_off = round_up(c_off + items * sizeof(int32_t), 256);
  const size_t total = p_off + items * ms * group_size(g) * (g->head_dim + 2) * sizeof(float);
  if (counters_off) *counters_off = c_off;
  if (part_off) *part_off = p_off;
  if (split_tokens) *split_tokens = st;
  if (max_splits) *max_splits = ms;
  return total;
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
  zp_status st = validate_geom(geom, "zp_paged_decode");
  if (st != ZP_OK) return st;
  if (!cache || !cache->k || !cache->v) return fail(ZP_EINVAL, "zp_paged_decode: cache K/V NULL");
  if (layer < 0 || layer >= geom->num_layers)
    return fail(ZP_EINVAL, "zp_paged_decode: layer %d out of range", layer);
  if (batch < 0 || table_stride <= 0 || max_seq_len < 0)
    return fail(ZP_EINVAL, "zp_paged_decode: bad batch/table_stride/max_seq_len");
  if (batch == 0) return ZP_OK;
  if (!q || !k_new || !v_new || !block_tables || !seq_lens || !out || !workspace)
    return fail(ZP_EINVAL, "zp_paged_decode: NULL buffer");
  if (qslot && !cache->qwin) return fail(ZP_EINVAL, "zp_paged_decode: qslot given but qwin NULL");
  size_t c_off, p_off;
  int32_t split_tokens, max_splits;
  const size_t need =
      decode_ws_layout(geom, batch, max_seq_len, &c_off, &p_off, &split_tokens, &max_splits);
  if (workspace_bytes < need)
    return fail(ZP_EINVAL, "zp_paged_decode: workspace %zu bytes, need %zu", workspace_bytes, need);

  DecodeParams P{};
  P.q = q; P.k_new = k_new; P.v_new = v_new;
  P.kc = cache->k; P.vc = cache->v; P.qwin = cache->qwin;
  P.tables = block_tables; P.seq_lens = seq_lens; P.qslot = qslot;
  P.out = out; P.lse = lse;
  char* ws = static_cast<char*>(workspace);
  P.err = reinterpret_cast<uint32_t*>(ws);
  P.counters = reinterpret_cast<int32_t*>(ws + c_off);
  P.part = reinterpret_cast<float*>(ws + p_off);
  const int64_t d = geom->head_dim;
  P.kv_layer_off = int64_t(layer) * geom->num_blocks * geom->num_kv_heads * geom->block_size * d;
  P.qwin_layer_off = int64_t(layer) * geom->max_slots * geom->num_q_heads * geom->window * d;
  P.table_stride = table_stride; P.num_blocks = geom->num_blocks; P.b = geom->block_size;
  P.h_kv = geom->num_kv_heads; P.w = geom->window; P.max_slots = geom->max_slots;
  P.split_tokens = split_tokens; P.max_splits = max_splits; P.max_seq_len = max_seq_len;
  P.qk_scale = kLog2e / std::sqrt(float(d));

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
  if (e != hipSuccess) return fail(ZP_EHIP, "zp_paged_decode: launch failed: %s", hipGetErrorString(e));
  return ZP_OK;
}
