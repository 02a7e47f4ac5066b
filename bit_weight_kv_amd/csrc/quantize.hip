// Group-wise 4-bit min/max quantisation: weights at load time and the
// K/V of new tokens on append; plus the debug reconstruction.
//
// Method: FlexGen README (giters.com mirror), key features, "Extreme
// Compression" -- weights and the attention cache are stored in 4 bits.  The
// pages state only the bit width; the group size (64), min/max asymmetric
// range, fp16 {min, scale} metadata, IEEE fp32 arithmetic and round-half-to-
// even are this library's readings (see include/fq.h).
//
// Mapping: one group of 64 fp16 values (128 contiguous bytes) is held by 8
// consecutive lanes, 8 values (one 16-byte load) each.  A wave covers 8
// groups = 1 KiB of contiguous input, so loads and the 4-byte code stores are
// fully coalesced; min/max are reduced across the 8 lanes with xor shuffles.
// HBM traffic per element: 2 B read + 0.5 B codes + 1/16 B meta written.
#include "common.h"
#include "quant_group.h"

namespace fq {
namespace {

// Quantise this lane's 8 values of a 64-value group spread over lanes
// sub = 0..7 of an aligned 8-lane segment.  Returns the lane's 8 codes as
// nibbles (element 0 in bits 0..3) and the group's {min, scale} fp16 bits.
__device__ inline uint32_t quant_group_lane(const uint4 raw, uint32_t& meta_bits) {
  float v[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = h2f((uint16_t)(w[j] & 0xFFFFu));
    v[2 * j + 1] = h2f((uint16_t)(w[j] >> 16));
  }
  uint32_t packed[1];
  quant_group<8, 8>(v, packed, meta_bits);
  return packed[0];
}

__device__ inline uint4 load8(const uint16_t* p, bool aligned) {
  if (aligned) {  // read once: a non-temporal load
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  uint4 r;
  r.x = (uint32_t)p[0] | ((uint32_t)p[1] << 16);
  r.y = (uint32_t)p[2] | ((uint32_t)p[3] << 16);
  r.z = (uint32_t)p[4] | ((uint32_t)p[5] << 16);
  r.w = (uint32_t)p[6] | ((uint32_t)p[7] << 16);
  return r;
}

// Row-major matrix [rows, cols] (row stride ldx) -> packed codes/meta.  Each
// wave takes QG x 8 consecutive groups: load i of the wave covers groups
// 8 (QG w + i) .. +7 (1 KiB of contiguous input when rows are contiguous), and
// every lane issues its QG loads before quantising, so QG loads per lane are
// in flight.  CONTIG: ldx == cols, so group g starts at element 64 g.
template <bool ALIGNED, bool CONTIG, int QG>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* __restrict__ x, int64_t n_groups,
                                                            int64_t gpr, int64_t ldx, uint8_t* __restrict__ codes,
                                                            uint16_t* __restrict__ meta) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t wave = t >> 6;
  const int seg = (int)((t >> 3) & 7), sub = (int)(t & 7);
  uint4 raw[QG];
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    const int64_t g = (wave * QG + i) * 8 + seg;
    raw[i] = make_uint4(0, 0, 0, 0);
    if (g < n_groups) {
      const uint16_t* src;
      if (CONTIG) {
        src = x + g * 64 + sub * 8;
      } else {
        const int64_t r = g / gpr, c = g - r * gpr;
        src = x + r * ldx + c * 64 + sub * 8;
      }
      raw[i] = load8(src, ALIGNED);
    }
  }
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    const int64_t g = (wave * QG + i) * 8 + seg;
    uint32_t mb;
    const uint32_t packed = quant_group_lane(raw[i], mb);
    if (g < n_groups) {
      reinterpret_cast<uint32_t*>(codes + g * 32)[sub] = packed;
      if (sub == 0) reinterpret_cast<uint32_t*>(meta)[g] = mb;
    }
  }
}

// K/V of T new tokens -> cache positions pos..pos+T-1.  Groups enumerate
// (b, t, which, head, group-in-head) with the group index fastest.
template <bool ALIGNED>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                        int64_t ld, int64_t n_groups, int T, int H, int gpd,
                                                        int64_t b0, int64_t cap, int64_t pos,
                                                        uint8_t* __restrict__ kc, uint16_t* __restrict__ km,
                                                        uint8_t* __restrict__ vc, uint16_t* __restrict__ vm) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t g = t >> 3;
  const int sub = (int)(t & 7);
  const bool ok = g < n_groups;
  int64_t rest = ok ? g : 0;
  const int gi = (int)(rest % gpd);
  rest /= gpd;
  const int head = (int)(rest % H);
  rest /= H;
  const int which = (int)(rest & 1);
  rest >>= 1;
  const int tok = (int)(rest % T);
  const int64_t b = rest / T;
  const int d = gpd * 64;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (ok) {
    const uint16_t* src = (which ? v : k) + (b * T + tok) * ld + (int64_t)head * d + gi * 64 + sub * 8;
    raw = load8(src, ALIGNED);
  }
  uint32_t mb;
  const uint32_t packed = quant_group_lane(raw, mb);
  if (ok) {
    const int64_t row = ((b0 + b) * H + head) * cap + pos + tok;
    uint8_t* codes = which ? vc : kc;
    uint16_t* meta = which ? vm : km;
    reinterpret_cast<uint32_t*>(codes + row * (d / 2) + gi * 32)[sub] = packed;
    if (sub == 0) reinterpret_cast<uint32_t*>(meta)[row * gpd + gi] = mb;
  }
}

// fp16 cache: K/V of T new tokens copied unchanged to positions pos..pos+T-1.
// Items enumerate (b, t, which, head, 8-channel chunk) with the chunk fastest,
// one 16-byte store per thread.
template <bool ALIGNED>
__global__ __launch_bounds__(256) void kv_append_f16_kernel(const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v, int64_t ld,
                                                            int64_t n_items, int T, int H, int cpd, int64_t b0,
                                                            int64_t cap, int64_t pos, uint16_t* __restrict__ k16,
                                                            uint16_t* __restrict__ v16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_items) return;
  int64_t rest = i;
  const int c = (int)(rest % cpd);
  rest /= cpd;
  const int head = (int)(rest % H);
  rest /= H;
  const int which = (int)(rest & 1);
  rest >>= 1;
  const int tok = (int)(rest % T);
  const int64_t b = rest / T;
  const int d = cpd * 8;
  const uint4 raw = load8((which ? v : k) + (b * T + tok) * ld + (int64_t)head * d + c * 8, ALIGNED);
  const int64_t row = ((b0 + b) * H + head) * cap + pos + tok;
  reinterpret_cast<uint4*>((which ? v16 : k16) + row * d)[c] = raw;
}

// y = fp16(min + code * s) with one rounding (fused fp16 multiply-add).
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ meta, int64_t n8,
                                                      uint16_t* __restrict__ y) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;
  const uint32_t w = reinterpret_cast<const uint32_t*>(codes)[t];
  const uint32_t mb = reinterpret_cast<const uint32_t*>(meta)[t >> 3];  // 8 words of 8 codes per group
  const half_t mn = __builtin_bit_cast(half_t, (uint16_t)(mb & 0xFFFF));
  const half_t s = __builtin_bit_cast(half_t, (uint16_t)(mb >> 16));
  uint16_t out[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const half_t c = (half_t)(float)((w >> (4 * j)) & 0xF);
    out[j] = __builtin_bit_cast(uint16_t, __builtin_fmaf16(c, s, mn));
  }
  uint4 r;
  r.x = out[0] | ((uint32_t)out[1] << 16);
  r.y = out[2] | ((uint32_t)out[3] << 16);
  r.z = out[4] | ((uint32_t)out[5] << 16);
  r.w = out[6] | ((uint32_t)out[7] << 16);
  reinterpret_cast<uint4*>(y)[t] = r;
}

}  // namespace

fq_status launch_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                               uint16_t* meta, hipStream_t st) {
  const int64_t gpr = cols / 64;
  const int64_t n_groups = rows * gpr;
  if (n_groups == 0) return FQ_OK;
  constexpr int QG = 8;  // groups per 8-lane segment
  const int64_t blocks = ceil_div(ceil_div(n_groups, 8 * QG), 4);  // 4 waves per block
  const bool aligned = ((uintptr_t)x % 16 == 0) && (ldx % 8 == 0);
  const dim3 grid((unsigned)blocks), block(256);
  if (aligned && ldx == cols)
    quantize_rows_kernel<true, true, QG><<<grid, block, 0, st>>>(x, n_groups, gpr, ldx, codes, meta);
  else if (aligned)
    quantize_rows_kernel<true, false, QG><<<grid, block, 0, st>>>(x, n_groups, gpr, ldx, codes, meta);
  else
    quantize_rows_kernel<false, false, QG><<<grid, block, 0, st>>>(x, n_groups, gpr, ldx, codes, meta);
  return launch_check("quantize_rows_kernel");
}

}  // namespace fq

using namespace fq;

extern "C" fq_status fq_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const fq_packed* out,
                                 void* stream) {
  clear_error();
  FQ_CHECK_ARG(out != nullptr, "fq_quantize: out is NULL");
  if (out->group != FQ_GROUP) return fail(FQ_ERR_UNSUPPORTED, "fq_quantize: only group 64 is implemented");
  FQ_CHECK_ARG(rows >= 0 && cols >= 0, "fq_quantize: negative shape");
  FQ_CHECK_ARG(cols % 64 == 0, "fq_quantize: cols must be a multiple of 64");
  FQ_CHECK_ARG(ldx >= cols, "fq_quantize: ldx < cols");
  FQ_CHECK_ARG(out->rows == rows && out->cols == cols, "fq_quantize: out shape differs from input shape");
  if (rows == 0 || cols == 0) return FQ_OK;
  FQ_CHECK_ARG(x && out->codes && out->meta, "fq_quantize: NULL buffer");
  FQ_CHECK_ARG((uintptr_t)out->codes % 4 == 0 && (uintptr_t)out->meta % 4 == 0,
               "fq_quantize: codes/meta must be 4-byte aligned");
  hipStream_t st = as_stream(stream);
  const int tk = timing_begin(FQ_KC_QUANTIZE, st);
  FQ_TRY(launch_quantize_rows(x, rows, cols, ldx, out->codes, out->meta, st));
  timing_end(tk, FQ_KC_QUANTIZE, 0.0, (double)rows * cols * (2.0 + 0.5625), st);
  return FQ_OK;
}

extern "C" fq_status fq_dequantize(const fq_packed* in, uint16_t* y, void* stream) {
  clear_error();
  FQ_CHECK_ARG(in != nullptr, "fq_dequantize: in is NULL");
  if (in->group != FQ_GROUP) return fail(FQ_ERR_UNSUPPORTED, "fq_dequantize: only group 64 is implemented");
  FQ_CHECK_ARG(in->rows >= 0 && in->cols >= 0 && in->cols % 64 == 0, "fq_dequantize: bad shape");
  const int64_t n8 = in->rows * in->cols / 8;
  if (n8 == 0) return FQ_OK;
  FQ_CHECK_ARG(in->codes && in->meta && y, "fq_dequantize: NULL buffer");
  FQ_CHECK_ARG((uintptr_t)y % 16 == 0, "fq_dequantize: y must be 16-byte aligned");
  dequant_kernel<<<dim3((unsigned)ceil_div(n8, 256)), dim3(256), 0, as_stream(stream)>>>(in->codes, in->meta, n8, y);
  return launch_check("dequant_kernel");
}

extern "C" fq_status fq_kv_append(const fq_kv_layer* kv, const uint16_t* k, const uint16_t* v, int64_t ld,
                                  int64_t b0, int64_t B, int64_t T, int64_t pos, void* stream) {
  clear_error();
  FQ_CHECK_ARG(kv != nullptr, "fq_kv_append: kv is NULL");
  if (kv->group != FQ_GROUP) return fail(FQ_ERR_UNSUPPORTED, "fq_kv_append: only group 64 is implemented");
  FQ_CHECK_ARG(kv->head_dim > 0 && kv->head_dim % 64 == 0, "fq_kv_append: head_dim must be a multiple of 64");
  FQ_CHECK_ARG(b0 >= 0 && B >= 0 && T >= 0 && pos >= 0, "fq_kv_append: negative index");
  FQ_CHECK_ARG(b0 + B <= kv->batch, "fq_kv_append: sequence range exceeds the cache batch");
  FQ_CHECK_ARG(pos + T <= kv->capacity, "fq_kv_append: positions exceed the cache capacity");
  FQ_CHECK_ARG(ld >= (int64_t)kv->heads * kv->head_dim, "fq_kv_append: ld < heads*head_dim");
  FQ_CHECK_ARG(kv_bits_valid(*kv), "fq_kv_append: bits must be 4 or 16");
  if (B == 0 || T == 0) return FQ_OK;
  const bool aligned = ((uintptr_t)k % 16 == 0) && ((uintptr_t)v % 16 == 0) && (ld % 8 == 0);
  hipStream_t st = as_stream(stream);
  if (kv_is_f16(*kv)) {
    FQ_CHECK_ARG(k && v && kv->k16 && kv->v16, "fq_kv_append: NULL buffer");
    FQ_CHECK_ARG((uintptr_t)kv->k16 % 16 == 0 && (uintptr_t)kv->v16 % 16 == 0,
                 "fq_kv_append: fp16 cache must be 16-byte aligned");
    const int cpd = kv->head_dim / 8;
    const int64_t n_items = B * T * 2 * kv->heads * cpd;
    const dim3 grid((unsigned)ceil_div(n_items, 256));
    const int tk = timing_begin(FQ_KC_KV_APPEND, st);
    if (aligned)
      kv_append_f16_kernel<true><<<grid, dim3(256), 0, st>>>(k, v, ld, n_items, (int)T, kv->heads, cpd, b0,
                                                             kv->capacity, pos, kv->k16, kv->v16);
    else
      kv_append_f16_kernel<false><<<grid, dim3(256), 0, st>>>(k, v, ld, n_items, (int)T, kv->heads, cpd, b0,
                                                              kv->capacity, pos, kv->k16, kv->v16);
    FQ_TRY(launch_check("kv_append_f16_kernel"));
    timing_end(tk, FQ_KC_KV_APPEND, 0.0, (double)n_items * 8 * 4.0, st);
    return FQ_OK;
  }
  FQ_CHECK_ARG(k && v && kv->k_codes && kv->k_meta && kv->v_codes && kv->v_meta, "fq_kv_append: NULL buffer");
  const int gpd = kv->head_dim / 64;
  const int64_t n_groups = B * T * 2 * kv->heads * gpd;
  const dim3 grid((unsigned)ceil_div(n_groups * 8, 256));
  const int tk = timing_begin(FQ_KC_KV_APPEND, st);
  if (aligned)
    kv_append_kernel<true><<<grid, dim3(256), 0, st>>>(k, v, ld, n_groups, (int)T, kv->heads, gpd, b0, kv->capacity,
                                                       pos, kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta);
  else
    kv_append_kernel<false><<<grid, dim3(256), 0, st>>>(k, v, ld, n_groups, (int)T, kv->heads, gpd, b0, kv->capacity,
                                                        pos, kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta);
  FQ_TRY(launch_check("kv_append_kernel"));
  timing_end(tk, FQ_KC_KV_APPEND, 0.0, (double)n_groups * 64 * (2.0 + 0.5625), st);
  return FQ_OK;
}
