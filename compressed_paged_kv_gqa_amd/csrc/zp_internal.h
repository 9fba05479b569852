// Internal helpers shared by the host-side translation units of libzp.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "zp.h"

namespace zp {

// Records a formatted message for zp_last_error() on the calling thread and
// returns `st`, so callers can write `return fail(ZP_EINVAL, "...")`.
zp_status fail(zp_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

}  // namespace zp

namespace zp {

// Geometry checks shared by the GPU entry points (host-side, no HIP).
zp_status validate_geom(const zp_geom* g, const char* who);
inline int64_t elem_size(const zp_geom* g) { return g->dtype == ZP_DTYPE_BF16 ? 2 : 4; }
inline int32_t group_size(const zp_geom* g) { return g->num_q_heads / g->num_kv_heads; }

constexpr size_t kWsHeader = 256;  // bytes; first uint32 = device error bits
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Waves per SIMD the decode kernel's register budget is sized for (the
// occupancy it is compiled for), by element size, head dim and group size.
constexpr int decode_waves_per_simd(int elem_bytes, int d, int g) {
  return (elem_bytes == 2 && g <= 4) || (d == 64 && g <= 4) ? 3 : 2;
}

// Launch shape of one decode call: returns the tokens one workgroup covers
// (split-K granularity; a sequence longer than that is split and merged by
// a second kernel) and sets *waves, the wavefronts per workgroup.
int32_t decode_launch_shape(const zp_geom* g, int32_t batch, int32_t max_seq_len,
                            int32_t* waves);

}  // namespace zp
