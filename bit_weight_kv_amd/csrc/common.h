// Internal helpers shared by the libfq translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "fq.h"

namespace fq {

// ---- error reporting -------------------------------------------------------
void set_error(const std::string& msg);
void clear_error();
fq_status fail(fq_status s, const std::string& msg);
fq_status hip_fail(hipError_t e, const char* what);

#define FQ_CHECK_ARG(cond, msg)                                   \
  do {                                                            \
    if (!(cond)) return ::fq::fail(FQ_ERR_INVALID, (msg));        \
  } while (0)

#define FQ_HIP(call)                                              \
  do {                                                            \
    hipError_t fq_e_ = (call);                                    \
    if (fq_e_ != hipSuccess) return ::fq::hip_fail(fq_e_, #call); \
  } while (0)

#define FQ_TRY(call)                                              \
  do {                                                            \
    fq_status fq_s_ = (call);                                     \
    if (fq_s_ != FQ_OK) return fq_s_;                             \
  } while (0)

// Check for a launch error right after a kernel launch.
inline fq_status launch_check(const char* kernel) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, kernel);
  return FQ_OK;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Storage format of a KV-cache layer view: true for the fp16 cache, false for
// the 4-bit one (bits 4, or 0 in a zero-initialised view).
inline bool kv_is_f16(const fq_kv_layer& kv) { return kv.bits == 16; }
inline bool kv_bits_valid(const fq_kv_layer& kv) { return kv.bits == 0 || kv.bits == 4 || kv.bits == 16; }

// ---- device vector types ---------------------------------------------------
typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

__device__ inline float h2f(uint16_t b) { return (float)__builtin_bit_cast(half_t, b); }
__device__ inline uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (half_t)f); }

// ---- per-launch timing (timing.hip) -----------------------------------------
// timing_begin returns a token (or -1 when timing is off, the class is not
// selected, or the event pool is exhausted); timing_end closes it.
int timing_begin(int cls, hipStream_t st);
void timing_end(int token, int cls, double flops, double bytes, hipStream_t st);

// ---- internal launchers used across translation units ----------------------
fq_status launch_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                               uint16_t* meta, hipStream_t st);
fq_status launch_synth_normal(uint16_t* dst, int64_t n, uint64_t seed, uint64_t stream_id, int64_t first,
                              double sigma, hipStream_t st);
fq_status launch_fill_f16(uint16_t* dst, int64_t n, uint16_t value, hipStream_t st);
fq_status launch_embed(const int32_t* ids, int64_t rows, int64_t T, int64_t pos0, const uint16_t* emb,
                       const uint16_t* posemb, int64_t h, uint16_t* x, hipStream_t st);
fq_status launch_argmax(const float* logits, int64_t B, int64_t V, int64_t ld, int32_t* out, hipStream_t st);
fq_status launch_gather_rows(const uint16_t* x, int64_t B, int64_t T, int64_t h, uint16_t* y, hipStream_t st);

}  // namespace fq
