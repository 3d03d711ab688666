// Host-side helpers shared by the C ABI's source files: the thread-local
// error message, argument checks, sizes and the RoPE frequency table.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "c2kv.h"
#include "c2kv_device.hpp"

namespace c2kv {
namespace host {

// Set the calling thread's error message; returns s.
c2kv_status fail(c2kv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the message; returns C2KV_OK.
c2kv_status ok();
c2kv_status hip_fail(hipError_t e, const char* what);
const char* last_error();

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t elem_bytes(c2kv_dtype dt) { return dt == C2KV_BF16 ? 2 : 4; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }
inline int32_t num_slots_i(int32_t n, int32_t k) { return (n + k - 1) / k; }

// hq, hkv, head_dim and dtype supported by the kernels
c2kv_status check_heads(int32_t hq, int32_t hkv, int32_t head_dim, c2kv_dtype dt);
c2kv_status check_theta(float theta);
// a device pointer: non-NULL and 16-byte aligned
c2kv_status check_dev(const void* p, const char* name);
// a workspace of at least `need` bytes, 256-byte aligned (none needed: OK)
c2kv_status check_ws(void* ws, size_t ws_bytes, size_t need);
// inv_freq_i = theta^(-2i/d) in double, rounded once to float
RopeFreqs make_freqs(int head_dim, float theta);
// log2(e) / sqrt(head_dim): the softmax scale in the exp2 domain
float scale_log2(int head_dim);

}  // namespace host
}  // namespace c2kv
