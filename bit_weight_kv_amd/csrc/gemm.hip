// Dequant-fused projection GEMM and its fp16-weight variant:
//   C[M, N] = epilogue(A[M, K] * W^T),  A fp16 row-major, W [N, K].
//
// The compressed weight is the 4-bit group format (groups of 64 along K, fp16
// {min, scale} per group; FlexGen README, "Extreme Compression").  Compute
// runs on the reconstructed fp16 weight with fp32 accumulation on the gfx950
// matrix cores (v_mfma_f32_16x16x32_f16).
//
// Tiling (one K step = 64 = exactly one quantisation group per weight row):
//   * a block of WM x WN waves owns a BM x BN tile of C;
//   * per K step the block stages A[BM, 64] (fp16) and the reconstructed
//     W[BN, 64] (fp16) in LDS, double-buffered, rows padded to 72 halves so
//     the 16-lane fragment reads hit distinct banks;
//   * the 4-bit codes are read from HBM as 16-byte vectors (32 codes), turned
//     into fp16 with the exponent trick (0x6400 | code is the fp16 value
//     1024 + code, exact) and reconstructed with one packed fp16 FMA, which
//     rounds min + code * s once -- bit-identical to the reference
//     reconstruction;
//   * each wave runs (BM/WM/16) x (BN/WN/16) MFMA tiles per 32-wide k slice.
// Blocks are remapped so that neighbouring M tiles of one N tile share an XCD
// (the hardware deals consecutive block ids round-robin to the 8 XCDs, each
// with its own L2), so one XCD's L2 serves all re-reads of a weight tile.
// Split-K (grid.z) writes fp32 partials that a second kernel reduces and
// passes through the epilogue; used when the M x N grid cannot fill 256 CUs.
#include <cstdlib>
#include <mutex>
#include <string>
#include <type_traits>
#include <utility>

#include "common.h"
#include "quant_group.h"

namespace fq {
namespace {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // halves per staged row (144 bytes)

struct Epilogue {
  const uint16_t* bias;
  const uint16_t* residual;
  int64_t ldr;
  uint32_t flags;
  float qscale;
  int64_t qcols;
  void* C;
  int64_t ldc;
};

__device__ inline void epilogue_store(const Epilogue& e, int64_t m, int64_t n, float v) {
  if (e.flags & FQ_EPI_BIAS) v += h2f(e.bias[n]);
  if ((e.flags & FQ_EPI_QSCALE) && n < e.qcols) v *= e.qscale;
  if (e.flags & FQ_EPI_RELU) v = fmaxf(v, 0.0f);
  if (e.flags & FQ_EPI_RESIDUAL) v += h2f(e.residual[m * e.ldr + n]);
  if (e.flags & FQ_EPI_F32OUT)
    reinterpret_cast<float*>(e.C)[m * e.ldc + n] = v;
  else
    reinterpret_cast<uint16_t*>(e.C)[m * e.ldc + n] = f2h(v);
}

// K/V append fused into the epilogue of the QKV projection: columns
// [h, 2h) are keys and [2h, 3h) values; row m is token m % T of sequence
// b0 + m / T and lands at cache position pos + m % T.  fp16 storage (f16) or
// 4-bit groups of 64 channels, quantised exactly as the append kernel does.
struct KvAppend {
  uint8_t* kc;
  uint16_t* km;
  uint8_t* vc;
  uint16_t* vm;
  uint16_t* k16;
  uint16_t* v16;
  int64_t h, cap, b0, pos;
  int T, H, d, f16;
};

// Whether epilogue_store8 may use 16-byte accesses for every 8-column chunk
// that lies inside N (C, residual and bias rows 16-byte aligned).
__device__ inline bool epilogue_vec_ok(const Epilogue& e) {
  const bool c_ok = e.ldc % 8 == 0 && (uintptr_t)e.C % 16 == 0;
  const bool r_ok = !(e.flags & FQ_EPI_RESIDUAL) || (e.ldr % 8 == 0 && (uintptr_t)e.residual % 16 == 0);
  const bool b_ok = !(e.flags & FQ_EPI_BIAS) || (uintptr_t)e.bias % 16 == 0;
  return c_ok && r_ok && b_ok;
}

// epilogue_store of v[0..7] at (m, n..n+7): the same arithmetic per element,
// with 16-byte loads and stores when `vec` and the chunk lies inside N.
__device__ inline void epilogue_store8(const Epilogue& e, int64_t m, int64_t n, const float* v, int64_t N,
                                       bool vec) {
  if (!vec || n + 8 > N) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (n + k < N) epilogue_store(e, m, n + k, v[k]);
    return;
  }
  float w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = v[k];
  if (e.flags & FQ_EPI_BIAS) {
    const uint4 b = *reinterpret_cast<const uint4*>(e.bias + n);
    const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] += h2f((uint16_t)(bw[k >> 1] >> (16 * (k & 1))));
  }
  if (e.flags & FQ_EPI_QSCALE) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (n + k < e.qcols) w[k] *= e.qscale;
  }
  if (e.flags & FQ_EPI_RELU) {
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = fmaxf(w[k], 0.0f);
  }
  if (e.flags & FQ_EPI_RESIDUAL) {
    const uint4 r = *reinterpret_cast<const uint4*>(e.residual + m * e.ldr + n);
    const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] += h2f((uint16_t)(rw[k >> 1] >> (16 * (k & 1))));
  }
  if (e.flags & FQ_EPI_F32OUT) {
    float4* c = reinterpret_cast<float4*>(reinterpret_cast<float*>(e.C) + m * e.ldc + n);
    c[0] = make_float4(w[0], w[1], w[2], w[3]);
    c[1] = make_float4(w[4], w[5], w[6], w[7]);
  } else {
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = (uint32_t)f2h(w[2 * k]) | (uint32_t)f2h(w[2 * k + 1]) << 16;
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(e.C) + m * e.ldc + n) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// 8 codes (one 32-bit word, element 2k in the low nibble of byte k) -> 8 fp16
// values fp16(mn + c*s) in natural order, as 4 packed pairs.  Pair j comes
// from byte j alone: the byte duplicated into halves 0 and 1 (a byte
// permute), then one AND-OR keeps the low nibble under exponent 0x64 (1024 + c,
// ulp 1) and the high nibble, still at bits 4..7, under exponent 0x54
// (64 + c: at that exponent bit 4 is worth 1); an exact fp16 subtract of
// {1024, 64} leaves the two codes, and one packed fp16 FMA rounds c*s + mn once.
__device__ inline void dequant8(uint32_t w, half2_t mn2, half2_t s2, uint32_t out[4]) {
  const half2_t bias = {(half_t)-1024.0f, (half_t)-64.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sel = 0x0C000C00u | (uint32_t)j << 16 | (uint32_t)j;  // bytes {b_j, 0, b_j, 0}
    const uint32_t p = (__builtin_amdgcn_perm(w, w, sel) & 0x00F0000Fu) | 0x54006400u;
    const half2_t c = __builtin_bit_cast(half2_t, p) + bias;  // exact: small integers
    out[j] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c, s2, mn2));
  }
}

template <int BM, int BN, int WM, int WN, bool PACKED>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(const uint16_t* __restrict__ A, int64_t M, int64_t lda,
                                                             const uint8_t* __restrict__ codes,
                                                             const uint16_t* __restrict__ meta,
                                                             const uint16_t* __restrict__ w16, int64_t N, int64_t K,
                                                             int k_tiles_per_split, Epilogue epi,
                                                             float* __restrict__ partial) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
  constexpr int A_CHUNKS = BM * 8;  // 16-byte chunks of A per K step
  constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
  constexpr int B_CHUNKS = PACKED ? BN * 2 : BN * 8;
  constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDS_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

  // XCD-aware tile order: block ids b, b+8, b+16, ... run on one XCD; give
  // them consecutive logical tiles (M fastest, so they share weight tiles).
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t nblk = tiles_m * tiles_n;
  const int64_t bid = blockIdx.x;
  int64_t logical = bid;
  if (nblk >= 16) {
    const int64_t per_xcd = nblk / 8;
    const int64_t xcd = bid % 8, slot = bid / 8;
    if (bid < per_xcd * 8) logical = xcd * per_xcd + slot;
  }
  const int64_t m0 = (logical % tiles_m) * BM;
  const int64_t n0 = (logical / tiles_m) * BN;

  const int KT = (int)(K / BK);
  const int kt0 = blockIdx.z * k_tiles_per_split;
  const int kt1 = min(KT, kt0 + k_tiles_per_split);

  uint4 ra[A_PER_T];
  uint4 rb[B_PER_T];
  uint32_t rm[B_PER_T];

  auto load_tiles = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int c = tid + i * NT;
      ra[i] = make_uint4(0, 0, 0, 0);
      if (c < A_CHUNKS) {
        const int r = c >> 3, kc = c & 7;
        const int64_t m = m0 + r;
        if (m < M) ra[i] = *reinterpret_cast<const uint4*>(A + m * lda + (int64_t)kt * BK + kc * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int c = tid + i * NT;
      rb[i] = make_uint4(0, 0, 0, 0);
      rm[i] = 0;
      if (c < B_CHUNKS) {
        if (PACKED) {
          const int r = c >> 1, half = c & 1;
          const int64_t n = n0 + r;
          if (n < N) {
            rb[i] = *reinterpret_cast<const uint4*>(codes + n * (K / 2) + (int64_t)kt * 32 + half * 16);
            rm[i] = reinterpret_cast<const uint32_t*>(meta)[n * (K / 64) + kt];
          }
        } else {
          const int r = c >> 3, kc = c & 7;
          const int64_t n = n0 + r;
          if (n < N) rb[i] = *reinterpret_cast<const uint4*>(w16 + n * K + (int64_t)kt * BK + kc * 8);
        }
      }
    }
  };

  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int c = tid + i * NT;
      if (c < A_CHUNKS) {
        const int r = c >> 3, kc = c & 7;
        *reinterpret_cast<uint4*>(&As[buf][r * LDS_STRIDE + kc * 8]) = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int c = tid + i * NT;
      if (c < B_CHUNKS) {
        if (PACKED) {
          const int r = c >> 1, half = c & 1;
          const half_t mn = __builtin_bit_cast(half_t, (uint16_t)(rm[i] & 0xFFFF));
          const half_t s = __builtin_bit_cast(half_t, (uint16_t)(rm[i] >> 16));
          const half2_t mn2 = {mn, mn}, s2 = {s, s};
          const uint32_t w[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t o[4];
            dequant8(w[q], mn2, s2, o);
            *reinterpret_cast<uint4*>(&Bs[buf][r * LDS_STRIDE + half * 32 + q * 8]) = make_uint4(o[0], o[1], o[2], o[3]);
          }
        } else {
          const int r = c >> 3, kc = c & 7;
          *reinterpret_cast<uint4*>(&Bs[buf][r * LDS_STRIDE + kc * 8]) = rb[i];
        }
      }
    }
  };

  float4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};

  if (kt0 < kt1) {
    load_tiles(kt0);
    store_tiles(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      const bool more = kt + 1 < kt1;
      if (more) load_tiles(kt + 1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        half8_t af[FM], bf[FN];
        const int kofs = ks * 32 + 8 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = *reinterpret_cast<const half8_t*>(&As[cur][(wm * TM + i * 16 + (lane & 15)) * LDS_STRIDE + kofs]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bf[j] = *reinterpret_cast<const half8_t*>(&Bs[cur][(wn * TN + j * 16 + (lane & 15)) * LDS_STRIDE + kofs]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
      if (more) store_tiles(cur ^ 1);
      __syncthreads();
    }
  }

  // D layout of the 16x16 MFMA: lane holds column lane%16, rows 4*(lane/16)+r.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn * TN + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * TM + i * 16 + 4 * (lane >> 4) + r;
        if (m < M && n < N) {
          if (partial)
            partial[((int64_t)blockIdx.z * M + m) * N + n] = acc[i][j][r];
          else
            epilogue_store(epi, m, n, acc[i][j][r]);
        }
      }
    }
  }
}

// ---- large-M kernel ---------------------------------------------------------
// 256 x 128 block tile, 4 waves in 2 x 2, each wave 128 x 64 (8 x 4 MFMA
// 16x16x32 tiles, fp32 accumulators in AGPRs).  K step 64.
//   * Every global operand moves with direct global -> LDS copies
//     (global_load_lds, 16 bytes per lane, one wave instruction fills 1 KiB of
//     LDS: lane l -> byte 16 l), so the loop never waits on a VGPR load.
//   * A (and fp16 B) tiles: a wave instruction covers 8 rows x 8 16-byte
//     chunks; each lane fetches global chunk c ^ swz(r) of its row so LDS slot
//     (r, c) holds chunk c ^ swz(r) (conflict-free fragment reads).
//   * Packed B: the K step's codes (128 rows x 32 B) and {min, scale} land in
//     one of three code slots; between the MFMAs each thread reconstructs
//     16 code bytes of one row (two threads per row) into the fp16 B stage.
//   * Three LDS stages; iteration kt multiplies stage kt, reconstructs the
//     codes of step kt+2 into stage kt+2, and issues step kt+3's codes and
//     stage kt+2's A copies; the wait before the single barrier leaves only
//     this iteration's A (and fp16 B) copies in flight.
// Rows beyond M (and weight rows beyond N) are clamped to the last valid row:
// they are read but never stored.
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* gbl_void_ptr;

// LDS chunk swizzle.  Measured with the LDS bank-conflict counter on gfx950:
// chunk c ^ (r & 7) is conflict-free both for the MFMA fragment reads (lane l
// reads row l & 15, chunk l >> 4) and for the reconstructed-weight stores
// (lane l writes row l >> 1, chunk (l & 1) * 4 + q), whereas 144-byte padded
// rows cost ~30 % extra LDS cycles on the reads.
__device__ inline int swz(int r) { return r & 7; }

template <bool PACKED>
__global__ __launch_bounds__(256) void gemm_big_kernel(const uint16_t* __restrict__ A, int64_t M, int64_t lda,
                                                       const uint8_t* __restrict__ codes,
                                                       const uint16_t* __restrict__ meta,
                                                       const uint16_t* __restrict__ w16, int64_t N, int64_t K,
                                                       Epilogue epi) {
  constexpr int BMx = 256, BNx = 128, TM = 128, TN = 64, FM = 8, FN = 4;
  constexpr int ROWB = BK * 2;                  // bytes per staged row (128)
  constexpr int A_BYTES = BMx * ROWB;           // 32 KiB per stage
  constexpr int B_BYTES = BNx * ROWB;           // 16 KiB per stage
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int CODE_BYTES = BNx * 32 + BNx * 4;  // packed codes + {min, scale} of one K step
  constexpr int CODE_SLOTS = PACKED ? 3 : 0;
  constexpr int VM_ISSUE = PACKED ? 8 : 12;     // copies per wave per stage (A, plus fp16 B)
  // One LDS object per stage and per operand.  The compiler's wait insertion
  // tracks direct-to-LDS copies per object: an access to an object with no
  // copy in flight needs no wait, while any access to an object with one
  // does.  With the loop unrolled by three every stage is a compile-time
  // object, so reading stage kt never waits for the copies into stage kt+2.
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds0[A_BYTES], a_lds1[A_BYTES], a_lds2[A_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t b_lds0[B_BYTES], b_lds1[B_BYTES], b_lds2[B_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t c_lds0[PACKED ? CODE_BYTES : 16], c_lds1[PACKED ? CODE_BYTES : 16],
      c_lds2[PACKED ? CODE_BYTES : 16];
  auto a_st = [&](auto s) -> uint8_t* {
    constexpr int S = decltype(s)::value;
    return S == 0 ? a_lds0 : S == 1 ? a_lds1 : a_lds2;
  };
  auto b_st = [&](auto s) -> uint8_t* {
    constexpr int S = decltype(s)::value;
    return S == 0 ? b_lds0 : S == 1 ? b_lds1 : b_lds2;
  };
  auto c_st = [&](auto s) -> uint8_t* {
    constexpr int S = decltype(s)::value;
    return S == 0 ? c_lds0 : S == 1 ? c_lds1 : c_lds2;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // XCD-aware, grouped tile order: the 32 blocks an XCD runs at once cover
  // 4 M tiles x 8 N tiles, so each activation tile is re-read from that XCD's
  // L2 by 8 blocks (measured best of 1, 2, 4, 8, 16 M tiles per group).
  // (Tile ids are only remapped within the first 8*floor(n/8) blocks.)
  const int64_t tiles_m = (M + BMx - 1) / BMx, tiles_n = (N + BNx - 1) / BNx;
  const int64_t nblk = tiles_m * tiles_n;
  const int64_t bid = blockIdx.x;
  int64_t lid = bid;
  {
    const int64_t per_xcd = nblk / 8;
    if (bid < per_xcd * 8) lid = (bid % 8) * per_xcd + bid / 8;
  }
  constexpr int GM = 4;
  const int64_t group = lid / (GM * tiles_n);
  const int64_t first_m = group * GM;
  const int64_t gsize = min((int64_t)GM, tiles_m - first_m);
  const int64_t in_group = lid - group * GM * tiles_n;
  const int64_t mt = first_m + in_group % gsize;
  const int64_t nt = in_group / gsize;
  const int64_t m0 = mt * BMx, n0 = nt * BNx;
  const int KT = (int)(K / BK);

  // direct copies of 8-row x 128-byte blocks: lane -> (row, chunk)
  const int cp_r = lane >> 3, cp_c = lane & 7;
  const uint16_t* a_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * (4 * i + wave) + cp_r;
    const int64_t m = min(m0 + r, M - 1);
    a_src[i] = A + m * lda + (cp_c ^ swz(r)) * 8;
  }
  const uint16_t* b_src[PACKED ? 1 : 4];
  if (!PACKED) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * (4 * i + wave) + cp_r;
      const int64_t n = min(n0 + r, N - 1);
      b_src[i] = w16 + n * K + (cp_c ^ swz(r)) * 8;
    }
  }
  auto issue_stage = [&](auto s, int kt) {
    uint8_t* dst = a_st(s);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds((gbl_void_ptr)(a_src[i] + (int64_t)kt * BK),
                                       (lds_void_ptr)(dst + (4 * i + wave) * 1024), 16, 0, 0);
    if (!PACKED) {
      uint8_t* bdst = b_st(s);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds((gbl_void_ptr)(b_src[i] + (int64_t)kt * BK),
                                         (lds_void_ptr)(bdst + (4 * i + wave) * 1024), 16, 0, 0);
    }
  };
  // packed codes of one K step: wave w copies rows 32w..32w+31 (two lanes per
  // row), waves 0 and 1 also copy the meta of rows 64w..64w+63
  const int code_r = wave * 32 + (lane >> 1);
  const uint8_t* code_src = PACKED ? codes + min(n0 + code_r, N - 1) * (K / 2) + (lane & 1) * 16 : nullptr;
  const uint16_t* meta_src = PACKED ? meta + min(n0 + wave * 64 + lane, N - 1) * (K / 64) * 2 : nullptr;
  auto issue_codes = [&](auto s, int kt) {
    uint8_t* dst = c_st(s);
    __builtin_amdgcn_global_load_lds((gbl_void_ptr)(code_src + (int64_t)kt * 32), (lds_void_ptr)(dst + wave * 1024),
                                     16, 0, 0);
    if (wave < 2)
      __builtin_amdgcn_global_load_lds((gbl_void_ptr)(meta_src + (int64_t)kt * 2),
                                       (lds_void_ptr)(dst + BNx * 32 + wave * 256), 4, 0, 0);
  };
  // reconstruction: thread -> (row, 32-wide k half) of the B tile
  const int b_row = tid >> 1, b_half = tid & 1;
  uint4 cw = make_uint4(0, 0, 0, 0);
  uint32_t cm = 0;
  // explicit LDS reads (waited inside the asm block): the compiler would
  // otherwise wait for every direct copy in flight before reading a slot
  auto read_codes = [&](auto s) {
    const uint32_t base = (uint32_t)(uintptr_t)c_st(s);
    const uint32_t ca = base + b_row * 32 + b_half * 16, ma = base + BNx * 32 + b_row * 4;
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 v;
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b32 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v), "=&v"(cm)
        : "v"(ca), "v"(ma)
        : "memory");
    cw = make_uint4(v[0], v[1], v[2], v[3]);
  };
  auto store_b_part = [&](auto s, int q) {
    uint8_t* dst = b_st(s) + b_row * ROWB;
    const int c = b_half * 4 + q;
    const half_t mn = __builtin_bit_cast(half_t, (uint16_t)(cm & 0xFFFF));
    const half_t sc = __builtin_bit_cast(half_t, (uint16_t)(cm >> 16));
    const half2_t mn2 = {mn, mn}, s2 = {sc, sc};
    const uint32_t w = q == 0 ? cw.x : q == 1 ? cw.y : q == 2 ? cw.z : cw.w;
    uint32_t o[4];
    dequant8(w, mn2, s2, o);
    // Written with an explicit ds_write: the compiler cannot tell this store
    // from the direct copies in flight and would otherwise wait for all of
    // them here.  It targets a stage with no copy in flight; the barrier's
    // lgkmcnt(0) wait completes it before any wave reads the stage.
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = {o[0], o[1], o[2], o[3]};
    const uint32_t addr = (uint32_t)(uintptr_t)(dst + ((c ^ swz(b_row)) * 16));
    asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
  };

  float4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};

  // prologue: stages 0 and 1 complete, step 2's codes in slot 2
  if (PACKED) {
    if (KT > 0) issue_codes(I0{}, 0);
    if (KT > 1) issue_codes(I1{}, 1);
    if (KT > 2) issue_codes(I2{}, 2);
  }
  if (KT > 0) issue_stage(I0{}, 0);
  if (KT > 1) issue_stage(I1{}, 1);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  if (PACKED) {
    if (KT > 0) {
      read_codes(I0{});
#pragma unroll
      for (int q = 0; q < 4; ++q) store_b_part(I0{}, q);
    }
    if (KT > 1) {
      read_codes(I1{});
#pragma unroll
      for (int q = 0; q < 4; ++q) store_b_part(I1{}, q);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  const int fr = lane & 15;      // fragment row within a 16-row block
  const int fk = lane >> 4;      // 8-element k chunk within a 32-wide k slice
  // Iteration kt (stage S = kt % 3): reconstruct step kt+2's codes (slot
  // (S+2)%3) into B stage (S+2)%3 between the MFMAs, issue step kt+3's codes
  // into slot S and stage kt+2's A copies into A stage (S+2)%3.
  auto iteration = [&](auto s, int kt) {
    constexpr int S = decltype(s)::value;
    using S2 = std::integral_constant<int, (S + 2) % 3>;
    const bool pre = kt + 2 < KT;
    if (PACKED) read_codes(S2{});  // stale but harmless when kt+2 >= KT
    if (PACKED && kt + 3 < KT) issue_codes(s, kt + 3);
    if (pre) issue_stage(S2{}, kt + 2);
    const uint8_t* As_ = a_st(s);
    const uint8_t* Bs_ = b_st(s);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kc = ks * 4 + fk;
      half8_t bf[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * TN + j * 16 + fr;
        bf[j] = *reinterpret_cast<const half8_t*>(Bs_ + r * ROWB + ((kc ^ swz(r)) * 16));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * TM + i * 16 + fr;
        const half8_t af = *reinterpret_cast<const half8_t*>(As_ + r * ROWB + ((kc ^ swz(r)) * 16));
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[i][j], 0, 0, 0);
        // unconditional: once no stage is left to fill this rewrites a stage nobody reads
        if (PACKED && ks == 1 && (i & 1) == 1) store_b_part(S2{}, i >> 1);
      }
    }
    if (pre) {
      if (VM_ISSUE == 8)
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };
  for (int kt = 0; kt < KT; kt += 3) {
    iteration(I0{}, kt);
    if (kt + 1 < KT) iteration(I1{}, kt + 1);
    if (kt + 2 < KT) iteration(I2{}, kt + 2);
  }

#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn * TN + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * TM + i * 16 + 4 * (lane >> 4) + r;
        if (m < M && n < N) epilogue_store(epi, m, n, acc[i][j][r]);
      }
    }
  }
}

// Direct global -> LDS copies written as inline asm.  The compiler then sees
// no LDS write in flight and inserts no waits of its own for them: the kernel
// that uses these orders every copy with explicit s_waitcnt + s_barrier.
// (Through the builtin, the compiler's per-object tracking of such copies
// falls back to waiting for all of them once a kernel has many copy sites.)
// M0 holds the wave-uniform LDS base; each lane's data lands at
// base + lane * size.  One wait state separates the M0 write from the copy.
// The copies are addressed as a wave-uniform 64-bit base (SGPRs) plus a
// 32-bit per-lane byte offset: half the per-lane address bytes, and a base
// that advances with scalar adds only.
__device__ inline void dma_lds16_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
__device__ inline void dma_lds4_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
// acc += a * b (16x16x32 fp16 MFMA) with the accumulator pinned to AGPRs
// (through the builtin, a wave holding 256 accumulators gets part of them
// assigned to VGPRs and copied around every MFMA), kept in program order
// relative to every other such MFMA (the compiler's scheduler would otherwise
// reorder them and wait for all fragment reads before the first one).  The
// compiler does not see these as MFMAs, so it inserts no wait between the
// last one and a read of its result: kernels end their MFMA chains with
// mfma_results_ready.
__device__ inline void mfma16x16x32_acc_ordered(float4_t& acc, const half8_t& a, const half8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// After the last MFMA of a chain: wait out the MFMA write -> VALU read
// latency (24 wait states, more than a 16x16x32 MFMA's 8 passes need) before
// the accumulators are read.  Nothing ties a compiler-generated register read
// to this statement, so the order is checked instead: a CPU test compiles
// this file to assembly and requires that no accumulator read, write or move
// lies between a kernel's first inline-asm MFMA and this wait, and that no
// such kernel spills.  (Binding the accumulators to empty statements after
// the wait made the register allocator move them before it.)
__device__ inline void mfma_results_ready() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Four MFMAs (acc_j += a * b_j) with the reconstruction of one 8-code word
// interleaved between them: a wave's VALU work overlaps its own MFMAs only
// when the two are interleaved finely (measured: 8 MFMAs + 16 independent
// VALU ops cost 162 cycles interleaved, 213 back to back, 147 for the MFMAs
// alone).  13 instructions per 8 weights: the even elements' nibbles masked
// into a byte word and the odd elements' shifted into another; two byte
// permutes pair them as elements {0,1,2,3} and {4,5,6,7}; the scaled fp8
// conversion turns each byte into an exact fp16 integer (as an OCP e4m3 value
// a byte c < 16 is c * 2^-9, so the scale 2^9 gives c); one packed fp16 FMA
// per pair rounds c*s + min once, with {min, scale} taken from the halves of
// `ms` -- the same values as dequant8.  Its outputs are consumed by later
// MFMAs only, never inside this block.
// General form: MFMA k computes c_k += a_k * b_k.
__device__ inline void mfma4_rebuild_ab(float4_t& c0, float4_t& c1, float4_t& c2, float4_t& c3, const half8_t& a0,
                                        const half8_t& a1, const half8_t& a2, const half8_t& a3, const half8_t& b0,
                                        const half8_t& b1, const half8_t& b2, const half8_t& b3, uint32_t w,
                                        uint32_t ms, half8_t& out) {
  // separate volatile statements keep their order; one accumulator per MFMA
  // statement keeps every accumulator in place (a statement binding several
  // makes the register allocator copy them around)
  uint32_t t, u, p0, p1, o0, o1, o2, o3;
  mfma16x16x32_acc_ordered(c0, a0, b0);
  asm volatile(
      "v_and_b32 %0, %3, %2\n\t"      // t: bytes {e0, e2, e4, e6}
      "v_lshrrev_b32 %1, 4, %2\n\t"
      "v_and_b32 %1, %3, %1"            // u: bytes {e1, e3, e5, e7}
      : "=&v"(t), "=&v"(u)
      : "v"(w), "s"(0x0F0F0F0Fu));
  mfma16x16x32_acc_ordered(c1, a1, b1);
  asm volatile(
      "v_perm_b32 %0, %3, %4, %5\n\t"  // bytes {e0, e1, e2, e3}
      "v_perm_b32 %1, %3, %4, %6\n\t"  // bytes {e4, e5, e6, e7}
      "v_cvt_scalef32_pk_f16_fp8 %2, %0, %7"
      : "=&v"(p0), "=&v"(p1), "=&v"(o0)
      : "v"(u), "v"(t), "s"(0x05010400u), "s"(0x07030602u), "s"(0x44000000u));  // 512.0f
  mfma16x16x32_acc_ordered(c2, a2, b2);
  asm volatile(
      "v_cvt_scalef32_pk_f16_fp8 %0, %3, %5 op_sel:[1,0,0]\n\t"
      "v_cvt_scalef32_pk_f16_fp8 %1, %4, %5\n\t"
      "v_cvt_scalef32_pk_f16_fp8 %2, %4, %5 op_sel:[1,0,0]"
      : "=&v"(o1), "=&v"(o2), "=&v"(o3)
      : "v"(p0), "v"(p1), "s"(0x44000000u));
  mfma16x16x32_acc_ordered(c3, a3, b3);
  asm volatile(
      "v_pk_fma_f16 %0, %0, %4, %4 op_sel:[0,1,0] op_sel_hi:[1,1,0]\n\t"
      "v_pk_fma_f16 %1, %1, %4, %4 op_sel:[0,1,0] op_sel_hi:[1,1,0]\n\t"
      "v_pk_fma_f16 %2, %2, %4, %4 op_sel:[0,1,0] op_sel_hi:[1,1,0]\n\t"
      "v_pk_fma_f16 %3, %3, %4, %4 op_sel:[0,1,0] op_sel_hi:[1,1,0]"
      : "+v"(o0), "+v"(o1), "+v"(o2), "+v"(o3)
      : "v"(ms));
  out = __builtin_bit_cast(half8_t, make_uint4(o0, o1, o2, o3));
}

// The same reconstruction spread over two groups of four MFMAs (at most 7
// VALU instructions beside each group): with one wave per SIMD the wave
// issues everything itself, and 13 instructions around 4 MFMAs crowd their
// issue slots.  The first half leaves the two paired byte words and the
// first converted pair in p0, p1, o0; the second half finishes into `out`.
__device__ inline void mfma4_rebuild_h1(float4_t& c0, float4_t& c1, float4_t& c2, float4_t& c3, const half8_t& a,
                                        const half8_t& b0, const half8_t& b1, const half8_t& b2, const half8_t& b3,
                                        uint32_t w, uint32_t& p0, uint32_t& p1, uint32_t& o0) {
  uint32_t t, u;
  mfma16x16x32_acc_ordered(c0, a, b0);
  asm volatile(
      "v_and_b32 %0, %3, %2\n\t"
      "v_lshrrev_b32 %1, 4, %2"
      : "=&v"(t), "=&v"(u)
      : "v"(w), "s"(0x0F0F0F0Fu));
  mfma16x16x32_acc_ordered(c1, a, b1);
  asm volatile("v_and_b32 %0, %1, %0" : "+v"(u) : "s"(0x0F0F0F0Fu));
  mfma16x16x32_acc_ordered(c2, a, b2);
  asm volatile(
      "v_perm_b32 %0, %2, %3, %4\n\t"
      "v_perm_b32 %1, %2, %3, %5"
      : "=&v"(p0), "=&v"(p1)
      : "v"(u), "v"(t), "s"(0x05010400u), "s"(0x07030602u));
  mfma16x16x32_acc_ordered(c3, a, b3);
  asm volatile("v_cvt_scalef32_pk_f16_fp8 %0, %1, %2" : "=&v"(o0) : "v"(p0), "s"(0x44000000u));
}
__device__ inline void mfma4_rebuild_h2(float4_t& c0, float4_t& c1, float4_t& c2, float4_t& c3, const half8_t& a,
                                        const half8_t& b0, const half8_t& b1, const half8_t& b2, const half8_t& b3,
                                        uint32_t p0, uint32_t p1, uint32_t o0, uint32_t ms, half8_t& out) {
  uint32_t o1, o2, o3;
  mfma16x16x32_acc_ordered(c0, a, b0);
  asm volatile(
      "v_cvt_scalef32_pk_f16_fp8 %0, %2, %4 op_sel:[1,0,0]\n\t"
      "v_cvt_scalef32_pk_f16_fp8 %1, %3, %4"
      : "=&v"(o1), "=&v"(o2)
      : "v"(p0), "v"(p1), "s"(0x44000000u));
  mfma16x16x32_acc_ordered(c1, a, b1);
  asm volatile(
      "v_cvt_scalef32_pk_f16_fp8 %0, %2, %3 op_sel:[1,0,0]\n\t"
      "v_pk_fma_f16 %1, %1, %4, %4 op_sel:[0,1,0] op_sel_hi:[1,1,0]"
      : "=&v"(o3), "+v"(o0)
      : "v"(p1), "s"(0x44000000u), "v"(ms));
  mfma16x16x32_acc_ordered(c2, a, b2);
  asm volatile(
      "v_pk_fma_f16 %0, %0, %2, %2 op_sel:[0,1,0] op_sel_hi:[1,1,0]\n\t"
      "v_pk_fma_f16 %1, %1, %2, %2 op_sel:[0,1,0] op_sel_hi:[1,1,0]"
      : "+v"(o1), "+v"(o2)
      : "v"(ms));
  mfma16x16x32_acc_ordered(c3, a, b3);
  asm volatile("v_pk_fma_f16 %0, %0, %1, %1 op_sel:[0,1,0] op_sel_hi:[1,1,0]" : "+v"(o3) : "v"(ms));
  out = __builtin_bit_cast(half8_t, make_uint4(o0, o1, o2, o3));
}

// One row's 16 accumulators of a K or V group (columns nw + cs .. nw + cs + 15
// of the 64-column group starting at nw): bias, one rounding to fp16 (the
// value the unfused path stores in C), then the fp16 cache store or the 4-bit
// group quantisation across the 4 lanes (cs = 0, 16, 32, 48) holding the row.
__device__ inline void kv_append_epilogue(const Epilogue& e, const KvAppend& kv, const float* src, int64_t m,
                                          int64_t nw, int cs) {
  float v[16];
#pragma unroll
  for (int c = 0; c < 16; c += 4) {
    const float4 x = *reinterpret_cast<const float4*>(src + c);
    v[c] = x.x, v[c + 1] = x.y, v[c + 2] = x.z, v[c + 3] = x.w;
  }
  if (e.flags & FQ_EPI_BIAS) {
#pragma unroll
    for (int c = 0; c < 16; c += 8) {
      const uint4 b = *reinterpret_cast<const uint4*>(e.bias + nw + cs + c);
      const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) v[c + k] += h2f((uint16_t)(bw[k >> 1] >> (16 * (k & 1))));
    }
  }
  uint32_t hw[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) hw[k] = (uint32_t)f2h(v[2 * k]) | (uint32_t)f2h(v[2 * k + 1]) << 16;
  const int64_t col = nw - kv.h;
  const bool is_v = col >= kv.h;
  const int64_t c2 = is_v ? col - kv.h : col;
  const int head = (int)(c2 / kv.d), ch = (int)(c2 % kv.d);  // ch: first channel of the group
  const int64_t b = m / kv.T, t = m - b * kv.T;
  const int64_t row = ((kv.b0 + b) * kv.H + head) * kv.cap + kv.pos + t;
  if (kv.f16) {
    uint4* dst = reinterpret_cast<uint4*>((is_v ? kv.v16 : kv.k16) + row * kv.d + ch + cs);
    dst[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    dst[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
    return;
  }
  float f[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    f[2 * k] = h2f((uint16_t)(hw[k] & 0xFFFF));
    f[2 * k + 1] = h2f((uint16_t)(hw[k] >> 16));
  }
  uint32_t packed[2], mb;
  quant_group<16, 4>(f, packed, mb);
  *reinterpret_cast<uint2*>((is_v ? kv.vc : kv.kc) + row * (kv.d / 2) + ch / 2 + cs / 2) =
      make_uint2(packed[0], packed[1]);
  if (cs == 0) reinterpret_cast<uint32_t*>(is_v ? kv.vm : kv.km)[row * (kv.d / 64) + ch / 64] = mb;
}

// ---- large-M kernel, one wave per SIMD, weight operand rebuilt in registers --
// 256 x 256 block tile, 4 waves side by side in N, each 256 x 64 (16 x 4 MFMA
// 16x16x32 tiles, 256 fp32 accumulators pinned to AGPRs), K step 64 (two
// MFMA k slices, one quantisation group) per barrier.
//   * A: four LDS stages of 256 rows x 128 bytes (16-byte chunk c of row r
//     at slot c ^ ((r / 2) & 7)); step kt+3's copies are issued during step
//     kt, one copy instruction per row block of MFMAs.
//   * codes: three slots of 256 rows x 32 code bytes (16-byte half c of row
//     r at slot c ^ ((r / 8) & 1)) + 256 {min, scale} pairs; step kt+3's
//     copies are issued during step kt.
//   * k order: slice ks of lane group g (lanes 16 g .. 16 g + 15) covers the
//     step's 8-element k chunk 2 g + ks on both operands, so a lane's two
//     code words of a step are adjacent (one 8-byte LDS read per column
//     block); with the two swizzles every 32 lanes of a fragment or code read
//     touch each LDS bank equally often.
//   * the weight operand never passes through LDS as fp16: each wave rebuilds
//     its own 64 weight rows x the next step's 64 k (8 code words per lane)
//     in registers, one rebuild carried by every 16 MFMAs; no two waves
//     rebuild the same weights.
//   * each wave reads every A fragment of the stage (32 per step), three
//     ahead of its MFMAs.
//   * one barrier per step; the wait before it leaves this step's copies in
//     flight, so the next step's A stage is complete one step early and its
//     first fragments are read before the barrier.
// No fp16 B tile in LDS (an earlier 8-wave design staged one, written once and
// read by every wave), and half the reconstruction work per flop of a 2 x 2
// arrangement of the same waves.
//
// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>): an
// unrolled loop whatever the optimiser decides (an array indexed by the loop
// variable stays in registers).
template <typename F, int... Is>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <bool KVA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w4_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t lda, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ meta, int64_t N, int64_t K, Epilogue epi, KvAppend kva) {
  constexpr int BMx = 256, BNx = 256, TN = 64, FM = 16, FN = 4, BKx = 64;
  constexpr int ROWB = BKx * 2;                                   // 128 bytes per staged A row
  constexpr int A_BYTES = BMx * ROWB;                             // 32 KiB
  constexpr int C_BYTES = BNx * 32;  // 8 KiB per code slot
  constexpr int M_BYTES = BNx * 16;  // {min, scale} of 4 steps per weight row: 4 KiB per buffer
  constexpr int SC = 3;
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds0[A_BYTES], a_lds1[A_BYTES], a_lds2[A_BYTES],
      a_lds3[A_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t c_lds[SC * C_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t m_lds[2 * M_BYTES];
  auto a_st = [&](auto s) -> uint8_t* {
    constexpr int S = decltype(s)::value;
    return S == 0 ? a_lds0 : S == 1 ? a_lds1 : S == 2 ? a_lds2 : a_lds3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave;
  const int fr = lane & 15, fk = lane >> 4;

  // XCD-aware grouped order: the 32 blocks an XCD runs at once cover 2 M
  // tiles x 16 N tiles (over the four OPT-175B prefill products measured
  // 1.0-1.4 % faster than 4 x 8, 2 % faster than 1 x 32, 7 % than 8 x 4)
  const int64_t tiles_m = (M + BMx - 1) / BMx, tiles_n = (N + BNx - 1) / BNx;
  const int64_t nblk = tiles_m * tiles_n;
  const int64_t bid = blockIdx.x;
  int64_t lid = bid;
  {
    const int64_t per_xcd = nblk / 8;
    if (bid < per_xcd * 8) lid = (bid % 8) * per_xcd + bid / 8;
  }
  constexpr int GM = 2;
  const int64_t group = lid / (GM * tiles_n);
  const int64_t first_m = group * GM;
  const int64_t gsize = min((int64_t)GM, tiles_m - first_m);
  const int64_t in_group = lid - group * GM * tiles_n;
  const int64_t m0 = (first_m + in_group % gsize) * BMx, n0 = (in_group / gsize) * BNx;
  const int KT = (int)(K / BKx);  // a multiple of 4

  // Copies, as a wave-uniform base (the block's first row and the step) plus
  // a fixed 32-bit byte offset per lane.  The wave index is read into a
  // scalar register once, so every LDS destination is scalar too.
  //   A: instruction q (0..31) fills rows 8q..8q+7 (lane -> row 8q + lane / 8,
  //   slot lane & 7 holding chunk slot ^ ((row / 2) & 7)); wave w issues
  //   q = w + 4t.
  //   codes: instruction p (0..7) fills rows 32p..32p+31 (lane -> row
  //   32p + lane / 2, slot lane & 1 holding half slot ^ ((row / 8) & 1));
  //   wave w issues p = w and w + 4.
  //   meta: wave w copies rows 64w..64w+63, 4 bytes per lane.
  // Rows beyond M or N are clamped to the last one: read, never stored.
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  const uint8_t* a_blk = reinterpret_cast<const uint8_t*>(A + m0 * lda);
  const uint8_t* c_blk = codes + n0 * (K / 2);
  const uint8_t* m_blk = reinterpret_cast<const uint8_t*>(meta + n0 * (K / 64) * 2);
  uint32_t a_off[8], c_off[2];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int r = 8 * (wave + 4 * t) + (lane >> 3);
    a_off[t] = (uint32_t)((min(m0 + r, M - 1) - m0) * lda * 2 + ((lane & 7) ^ ((r >> 1) & 7)) * 16);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 32 * (wave + 4 * t) + (lane >> 1);
    c_off[t] = (uint32_t)((min(n0 + r, N - 1) - n0) * (K / 2) + ((lane & 1) ^ ((r >> 3) & 1)) * 16);
  }
  const uint32_t m_off = (uint32_t)((min(n0 + 64 * wave + lane, N - 1) - n0) * (K / 64) * 4);
  const uint32_t m_base = (uint32_t)(uintptr_t)m_lds;
  const uint32_t c_base = (uint32_t)(uintptr_t)c_lds;
  auto issue_a = [&](auto s, int kt) {
    const uint32_t dst = (uint32_t)(uintptr_t)a_st(s) + swave * 1024;
#pragma unroll
    for (int t = 0; t < 8; ++t) dma_lds16_s(a_off[t], a_blk + (int64_t)kt * 128, dst + t * 4096);
  };
  auto issue_codes = [&](int kt) {
    const uint32_t dst = c_base + (kt % SC) * C_BYTES;
#pragma unroll
    for (int t = 0; t < 2; ++t) dma_lds16_s(c_off[t], c_blk + (int64_t)kt * 32, dst + (swave + 4 * t) * 1024);
  };
  // {min, scale} of steps 4g..4g+3 (16 bytes per weight row) into buffer g % 2
  auto issue_meta = [&](int g, int buf) {
    dma_lds16_s(m_off, m_blk + (int64_t)g * 16, m_base + buf * M_BYTES + swave * 1024);
  };
  // this lane's weight operand: column block j = weight row 64 wn + 16 j + fr,
  // slice ks = k chunk 2 fk + ks of the step (one code word), {min, scale} per row
  uint32_t cw[2][FN], cm[FN];
  auto read_codes = [&](int kt) {
    const uint8_t* slot = c_lds + (kt % SC) * C_BYTES;
    const uint8_t* mrow = m_lds + ((kt >> 2) & 1) * M_BYTES + (kt & 3) * 4;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wn * TN + j * 16 + fr;
      const uint2 w = *reinterpret_cast<const uint2*>(slot + row * 32 + (((fk >> 1) ^ ((row >> 3) & 1)) * 16) +
                                                      (fk & 1) * 8);
      cw[0][j] = w.x, cw[1][j] = w.y;
      cm[j] = *reinterpret_cast<const uint32_t*>(mrow + row * 16);
    }
  };
  auto rebuild = [&](int ks, int j) {
    const half_t mn = __builtin_bit_cast(half_t, (uint16_t)(cm[j] & 0xFFFF));
    const half_t sc = __builtin_bit_cast(half_t, (uint16_t)(cm[j] >> 16));
    const half2_t mn2 = {mn, mn}, s2 = {sc, sc};
    uint32_t o[4];
    dequant8(cw[ks][j], mn2, s2, o);
    return __builtin_bit_cast(half8_t, make_uint4(o[0], o[1], o[2], o[3]));
  };
  auto a_frag = [&](const uint8_t* As_, int ks, int i) {
    const int r = i * 16 + fr;
    return *reinterpret_cast<const half8_t*>(As_ + r * ROWB + (((2 * fk + ks) ^ ((r >> 1) & 7)) * 16));
  };

  float4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};

  // prologue: codes and A of steps 0..2; operand of step 0 rebuilt
  issue_codes(0);
  issue_codes(1);
  issue_codes(2);
  issue_meta(0, 0);
  issue_a(I0{}, 0);
  issue_a(I1{}, 1);
  issue_a(I2{}, 2);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  half8_t bA[2][FN], bB[2][FN];
  read_codes(0);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < FN; ++j) bA[ks][j] = rebuild(ks, j);
  // A fragments three slots ahead (slot = 16 ks + i) in a ring of 4: the
  // ring's size divides the 32 slots of a step, so slot s of every step
  // uses entry s % 4
  half8_t fa[4];
  fa[0] = a_frag(a_lds0, 0, 0);
  fa[1] = a_frag(a_lds0, 0, 1);
  fa[2] = a_frag(a_lds0, 0, 2);

  // step kt: A stage kt % 4 (S), operand in bA for even kt (P = 0), else bB.
  // Reads step kt+1's code words (their copies completed at the last
  // barrier), issues step kt+3's copies over the first 11 row-block slots
  // (slot = 16 ks + i; 11 per wave, so the wait before the barrier leaves
  // exactly this step's copies in flight), and rebuilds step kt+1's operand
  // into the other register set: rebuild r (slice r / 4, column block r % 4)
  // rides on the MFMAs of slots 4 + 3 r and 5 + 3 r (two halves), so the
  // code words have 4 slots to arrive.  The last three slots read the next step's first three
  // fragments (that stage is complete).  (each of the four calls is its own
  // instantiation: a step body inlined twice keeps the accumulators out of
  // registers)
  auto step = [&](auto s, int kt) {
    constexpr int S = decltype(s)::value;
    constexpr int P = S & 1;
    using S3 = std::integral_constant<int, (S + 3) % 4>;
    using S1 = std::integral_constant<int, (S + 1) % 4>;
    half8_t(&bcur)[2][FN] = P == 0 ? bA : bB;
    half8_t(&bnxt)[2][FN] = P == 0 ? bB : bA;
    const uint8_t* As_ = a_st(s);
    read_codes(kt + 1);  // stale but harmless past the last step
    // step kt+3's copies, clamped to the last step: past it they rewrite an
    // A stage and a code slot that no later step reads (each was last read
    // the step before), so the MFMA chain carries no branches
    const int kc = min(kt + 3, KT - 1);
    const uint8_t* a_step = a_blk + (int64_t)kc * 128;
    const uint8_t* c_step = c_blk + (int64_t)kc * 32;
    // (steps with kt % 4 == 0 also copy the {min, scale} of steps kt+4..kt+7)
    const int gm = min((kt >> 2) + 1, (KT >> 2) - 1);
    const uint32_t a_dst = (uint32_t)(uintptr_t)a_st(S3{}) + swave * 1024;
    const uint32_t c_dst = c_base + ((kt + 3) % SC) * C_BYTES;
    uint32_t sp0 = 0, sp1 = 0, so0 = 0;  // a reconstruction's values between its two slots
    static_for<2 * FM>([&](auto sc) {
      constexpr int SL = decltype(sc)::value;
      constexpr int ks = SL / FM, i = SL % FM;
      if constexpr (SL < 8) {
        dma_lds16_s(a_off[SL], a_step, a_dst + SL * 4096);
      } else if constexpr (SL < 10) {
        dma_lds16_s(c_off[SL - 8], c_step, c_dst + (swave + 4 * (SL - 8)) * 1024);
      } else if constexpr (SL == 10 && S == 0) {
        issue_meta(gm, ((kt >> 2) + 1) & 1);
      }
      constexpr int NX = SL + 3;
      fa[NX % 4] = NX < 2 * FM ? a_frag(As_, NX / FM, NX % FM) : a_frag(a_st(S1{}), 0, NX - 2 * FM);
      __builtin_amdgcn_sched_barrier(0);
      const half8_t& af = fa[SL % 4];
      if constexpr (SL >= 4 && (SL - 4) % 3 == 0 && (SL - 4) / 3 < 2 * FN) {
        constexpr int r = (SL - 4) / 3;
        mfma4_rebuild_h1(acc[i][0], acc[i][1], acc[i][2], acc[i][3], af, bcur[ks][0], bcur[ks][1], bcur[ks][2],
                         bcur[ks][3], cw[r / FN][r % FN], sp0, sp1, so0);
      } else if constexpr (SL >= 5 && (SL - 5) % 3 == 0 && (SL - 5) / 3 < 2 * FN) {
        constexpr int r = (SL - 5) / 3;
        half8_t nb;
        mfma4_rebuild_h2(acc[i][0], acc[i][1], acc[i][2], acc[i][3], af, bcur[ks][0], bcur[ks][1], bcur[ks][2],
                         bcur[ks][3], sp0, sp1, so0, cm[r % FN], nb);
        bnxt[r / FN][r % FN] = nb;
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) mfma16x16x32_acc_ordered(acc[i][j], af, bcur[ks][j]);
      }
    });
    if constexpr (S == 0)
      asm volatile("s_waitcnt vmcnt(11) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // the same LDS wait where the compiler sees it (already satisfied): it
    // then knows the prefetched fragments have arrived and adds no wait
    // before the next step's first MFMAs, which would also cover the code
    // reads issued after the barrier
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt unconstrained
  };
  for (int kt = 0; kt < KT; kt += 4) {
    step(I0{}, kt);
    step(I1{}, kt + 1);
    step(I2{}, kt + 2);
    step(I3{}, kt + 3);
  }
  // the last steps' copies land in stages the epilogue reuses
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  // the last MFMAs' results are read by VALU instructions below
  mfma_results_ready();

  // epilogue staged through LDS, 16 rows x 64 columns per wave at a time
  // (row stride 68 floats), wave w in half (w & 1) of A stage w / 2
  {
    constexpr int SROW = 68;
    float* stg = reinterpret_cast<float*>(((wave >> 1) == 0 ? a_lds0 : a_lds1) + (wave & 1) * 8192);
    const bool vec = epilogue_vec_ok(epi);
    const int rr = lane >> 2, cs = (lane & 3) * 16;
    static_for<FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) stg[(4 * (lane >> 4) + r) * SROW + j * 16 + (lane & 15)] = acc[i][j][r];
      __syncthreads();
      const int64_t m = m0 + i * 16 + rr;
      const int64_t nw = n0 + wn * TN;  // this wave's 64 columns: one quantisation group of one head
      if (KVA && nw >= kva.h && nw < N) {
        if (m < M) kv_append_epilogue(epi, kva, stg + rr * SROW + cs, m, nw, cs);
      } else if (m < M) {
        for (int c = 0; c < 16; c += 8) {
          const float4 lo = *reinterpret_cast<const float4*>(stg + rr * SROW + cs + c);
          const float4 hi = *reinterpret_cast<const float4*>(stg + rr * SROW + cs + c + 4);
          const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          epilogue_store8(epi, m, nw + cs + c, v, N, vec);
        }
      }
      __syncthreads();
    });
  }
}

// ---- small-M ("decode") kernel ------------------------------------------------
// For M <= 256 (one decode step of the whole batch) a block owns every row of
// C and 256 weight rows; each of its 4 waves owns 64 weight rows and all
// 16*MB rows of A, so the weights are read exactly once per K range and need
// no LDS: every lane reconstructs its own MFMA operand from 8 code bytes
// (the 16 k values it contributes to the two 32-wide slices of a K step) in
// registers.  The A tile of a K step is staged in LDS (double-buffered,
// swizzled 128-byte rows) and shared by the 4 waves.  Within a K step, slice
// ks of lane group g covers k chunk 2g+ks (the same mapping on both
// operands), so a lane's codes for a K step are 8 contiguous bytes.  Split-K
// across blocks (grid.y) fills the chip; partial sums go through the same
// reduction kernel as the tiled path.
template <int MB, bool PACKED>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const uint16_t* __restrict__ A, int64_t M, int64_t lda,
                                                          const uint8_t* __restrict__ codes,
                                                          const uint16_t* __restrict__ meta,
                                                          const uint16_t* __restrict__ w16, int64_t N, int64_t K,
                                                          int k_tiles_per_split, Epilogue epi,
                                                          float* __restrict__ partial) {
  constexpr int ROWS = MB * 16;
  constexpr int CHUNKS = ROWS * 8;               // 16-byte chunks of an A tile
  constexpr int PER_T = (CHUNKS + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][ROWS * 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int64_t n_wave = (int64_t)blockIdx.x * 256 + wave * 64;
  const int64_t m_base = (int64_t)blockIdx.z * ROWS;  // M beyond 16*MB rows: one block per row group
  const int KT = (int)(K / BK);
  const int kt0 = blockIdx.y * k_tiles_per_split;
  const int kt1 = min(KT, kt0 + k_tiles_per_split);

  // weight rows of this lane: n_wave + 16 j + l16, clamped (never stored beyond N)
  int64_t wrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wrow[j] = min(n_wave + j * 16 + l16, N - 1);

  uint4 ra[PER_T];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = tid + i * 256;
      ra[i] = make_uint4(0, 0, 0, 0);
      if (c < CHUNKS) {
        const int r = c >> 3, ch = c & 7;
        if (m_base + r < M)
          ra[i] = *reinterpret_cast<const uint4*>(A + (m_base + r) * lda + (int64_t)kt * BK + ch * 8);
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = tid + i * 256;
      if (c < CHUNKS) {
        const int r = c >> 3, ch = c & 7;
        *reinterpret_cast<uint4*>(&As[buf][r * 64 + ((ch ^ (r & 7)) * 8)]) = ra[i];
      }
    }
  };
  // weight operand registers for one K step: 4 rows x (8 bytes of codes + meta) or 4 x 32 bytes fp16
  uint2 wc[4];
  uint32_t wm[4];
  uint4 wf[4][2];
  auto load_w = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (PACKED) {
        wc[j] = *reinterpret_cast<const uint2*>(codes + wrow[j] * (K / 2) + (int64_t)kt * 32 + g4 * 8);
        wm[j] = reinterpret_cast<const uint32_t*>(meta)[wrow[j] * (K / 64) + kt];
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(w16 + wrow[j] * K + (int64_t)kt * BK + g4 * 16);
        wf[j][0] = src[0];
        wf[j][1] = src[1];
      }
    }
  };

  float4_t acc[MB][4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};

  if (kt0 < kt1) {
    load_a(kt0);
    load_w(kt0);
    store_a(0);
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      const bool more = kt + 1 < kt1;
      // this step's weight operands
      half8_t bf[2][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (PACKED) {
          const half_t mn = __builtin_bit_cast(half_t, (uint16_t)(wm[j] & 0xFFFF));
          const half_t sc = __builtin_bit_cast(half_t, (uint16_t)(wm[j] >> 16));
          const half2_t mn2 = {mn, mn}, s2 = {sc, sc};
          uint32_t o[4];
          dequant8(wc[j].x, mn2, s2, o);
          bf[0][j] = __builtin_bit_cast(half8_t, make_uint4(o[0], o[1], o[2], o[3]));
          dequant8(wc[j].y, mn2, s2, o);
          bf[1][j] = __builtin_bit_cast(half8_t, make_uint4(o[0], o[1], o[2], o[3]));
        } else {
          bf[0][j] = __builtin_bit_cast(half8_t, wf[j][0]);
          bf[1][j] = __builtin_bit_cast(half8_t, wf[j][1]);
        }
      }
      if (more) {
        load_a(kt + 1);
        load_w(kt + 1);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int ch = 2 * g4 + ks;  // k chunk of this lane in slice ks
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int r = i * 16 + l16;
          const half8_t af = *reinterpret_cast<const half8_t*>(&As[cur][r * 64 + ((ch ^ (r & 7)) * 8)]);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[ks][j], acc[i][j], 0, 0, 0);
        }
      }
      if (more) store_a(cur ^ 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n_wave + j * 16 + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m_base + i * 16 + 4 * g4 + r;
        if (m < M && n < N) {
          if (partial)
            partial[((int64_t)blockIdx.y * M + m) * N + n] = acc[i][j][r];
          else
            epilogue_store(epi, m, n, acc[i][j][r]);
        }
      }
    }
  }
}

// ---- 4-bit decode GEMM, two waves per SIMD ----------------------------------
// The fallback of the one-wave-per-SIMD decode kernel below, for K-step
// counts that are not a multiple of 4 or a {min, scale} array that is not
// 16-byte aligned.  A block owns 256 weight rows and every row of A (16*MB);
// per K step (64 = one quantisation group) it copies the step's A tile
// (swizzled 128-byte rows), its codes (256 rows x 32 B) and {min, scale}
// global -> LDS with direct copies into a ring of stages issued ahead, and
// each lane rebuilds its own MFMA B operand from 8 code bytes per weight row
// one step ahead.  8 waves of 32 weight rows each: two waves share a SIMD, so
// one wave's LDS and barrier waits overlap the other's MFMAs.  Per K step a wave runs 2 slices x MB row blocks x 2 MFMAs and
// rebuilds 4 operand words for the next step (its 2 rows x 2 slices), each
// carried by the 4 MFMAs of a pair of row blocks.
//
// META4: {min, scale} copied 4 steps at a time (16 bytes per weight row, a
// 2-buffer ring beside the stages) when every split starts on a multiple of 4
// steps, instead of 4 bytes per row each step.
template <int MB, bool META4>
__global__ __launch_bounds__(512) void gemm_decode8_kernel(const uint16_t* __restrict__ A, int64_t M, int64_t lda,
                                                           const uint8_t* __restrict__ codes,
                                                           const uint16_t* __restrict__ meta, int64_t N, int64_t K,
                                                           int k_tiles_per_split, Epilogue epi,
                                                           float* __restrict__ partial) {
  constexpr int ROWS = MB * 16;
  constexpr int NQ = ROWS / 8;                  // A copies per step (8 rows of 128 B each)
  constexpr int A_INSTR = (NQ + 7) / 8;         // per wave: waves below NQ % 8 (all when 0) issue A_INSTR,
  constexpr int EXTRA = NQ % 8 ? NQ % 8 : 8;    // the others one fewer
  // copies per wave per step: A, one of codes, one of {min, scale} (META4:
  // one every fourth step, counted separately)
  constexpr int PER = A_INSTR + (META4 ? 1 : 2), PER_LO = PER - (EXTRA < 8 ? 1 : 0);
  constexpr int A_BYTES = ROWS * 128, C_BYTES = 256 * 32, STAGE = A_BYTES + C_BYTES + (META4 ? 0 : 256 * 4);
  constexpr int M_BYTES = 256 * 16;
  constexpr int S = 4;
  static_assert(S * STAGE <= 160 * 1024, "LDS ring too large");
  static_assert(MB >= 4, "two pairs of row blocks per slice carry the reconstructions");
  static_assert((S - 3) * PER + 1 <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[S * STAGE + (META4 ? 2 * M_BYTES : 0)];
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  uint8_t* const mring = lds + S * STAGE;  // META4: group g's {min, scale} in buffer g % 2, 16 bytes per row

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int64_t n_blk = (int64_t)blockIdx.x * 256;
  const int64_t m_base = (int64_t)blockIdx.z * ROWS;
  const int KT = (int)(K / BK);
  const int kt0 = blockIdx.y * k_tiles_per_split;
  const int kt1 = min(KT, kt0 + k_tiles_per_split);

  // A copies: instruction q = wave + 8t (q < NQ) fills rows 8q..8q+7 (lane ->
  // row 8q + lane / 8, slot lane % 8 holding chunk slot ^ (row % 8)); rows
  // past M are clamped (read, never stored).  Every copy is addressed as a
  // wave-uniform base (the block's first row or weight row, plus the step)
  // and a fixed 32-bit byte offset per lane (the host keeps lda small
  // enough); the wave index sits in a scalar register.
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  const uint8_t* a_blk = reinterpret_cast<const uint8_t*>(A + m_base * lda);
  const uint8_t* c_blk = codes + n_blk * (K / 2);
  const uint8_t* m_blk = reinterpret_cast<const uint8_t*>(meta + n_blk * (K / 64) * 2);
  uint32_t a_off[A_INSTR];
#pragma unroll
  for (int t = 0; t < A_INSTR; ++t) {
    const int r = 8 * (wave + 8 * t) + (lane >> 3);
    a_off[t] = (uint32_t)((min(m_base + r, M - 1) - m_base) * lda * 2 + ((lane & 7) ^ (r & 7)) * 16);
  }
  const uint32_t c_off = (uint32_t)((min(n_blk + wave * 32 + (lane >> 1), N - 1) - n_blk) * (K / 2) + (lane & 1) * 16);
  const uint32_t m_off = (uint32_t)((min(n_blk + wave * 32 + (lane & 31), N - 1) - n_blk) * (K / 64) * 4);
  auto issue = [&](int kt, int slot) {
    const uint32_t st = lds_base + slot * STAGE;
#pragma unroll
    for (int t = 0; t < A_INSTR; ++t)
      if (t + 1 < A_INSTR || swave < EXTRA)
        dma_lds16_s(a_off[t], a_blk + (int64_t)kt * 128, st + (swave + 8 * t) * 1024);
    dma_lds16_s(c_off, c_blk + (int64_t)kt * 32, st + A_BYTES + swave * 32 * 32);
    if constexpr (META4) {
      if ((kt & 3) == 0 && lane < 32)
        dma_lds16_s(m_off, m_blk + (int64_t)(kt >> 2) * 16,
                    (uint32_t)(uintptr_t)mring + ((kt >> 2) & 1) * M_BYTES + swave * 512);
    } else {
      if (lane < 32) dma_lds4_s(m_off, m_blk + (int64_t)kt * 4, st + A_BYTES + C_BYTES + swave * 128);
    }
  };
  // this lane's weight rows: wave * 32 + 16 j + l16
  uint2 cw[2];
  uint32_t cm[2];
  auto read_codes = [&](int slot, int kt) {
    const uint8_t* st = lds + slot * STAGE + A_BYTES;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = wave * 32 + j * 16 + l16;
      cw[j] = *reinterpret_cast<const uint2*>(st + row * 32 + g4 * 8);
      if constexpr (META4)
        cm[j] = *reinterpret_cast<const uint32_t*>(mring + ((kt >> 2) & 1) * M_BYTES + row * 16 + (kt & 3) * 4);
      else
        cm[j] = *reinterpret_cast<const uint32_t*>(st + C_BYTES + row * 4);
    }
  };
  auto rebuild = [&](int j, int w, half8_t (&b)[2][2]) {
    const half_t mn = __builtin_bit_cast(half_t, (uint16_t)(cm[j] & 0xFFFF));
    const half_t sc = __builtin_bit_cast(half_t, (uint16_t)(cm[j] >> 16));
    const half2_t mn2 = {mn, mn}, s2 = {sc, sc};
    uint32_t o[4];
    dequant8(w ? cw[j].y : cw[j].x, mn2, s2, o);
    b[w][j] = __builtin_bit_cast(half8_t, make_uint4(o[0], o[1], o[2], o[3]));
  };

  float4_t acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};

  if (kt0 < kt1) {
    for (int t = 0; t < S - 1 && kt0 + t < kt1; ++t) issue(kt0 + t, t);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    half8_t bA[2][2], bB[2][2];
    read_codes(0, kt0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int w = 0; w < 2; ++w) rebuild(j, w, bA);
    // One K step: MFMAs on `bcur`, step kt+1's operand rebuilt into `bnxt`
    // by the row-block pairs (0, 1) and (2, 3) of each slice (slice ks
    // rebuilds word ks of rows 0 and 1).  PH = kt % 4 (META4) or kt % 2.
    // (each call is its own instantiation: a step body inlined twice keeps
    // the accumulators out of registers)
    auto step = [&](auto ph, int kt, half8_t (&bcur)[2][2], half8_t (&bnxt)[2][2]) {
      constexpr int PH = decltype(ph)::value;
      // copies in flight after the wait: those of step kt+2, which carry the
      // {min, scale} of its group when META4 and kt+2 is a multiple of 4
      constexpr int MX = (META4 && PH == 2) ? 1 : 0;
      const int it = kt - kt0, slot = it % S;
      if (kt > kt0) {
        // steps kt and kt+1 complete in every wave; step kt-1's slot free
        if (kt + S - 2 < kt1) {
          if (swave < EXTRA)
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((S - 3) * PER + MX) : "memory");
          else
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((S - 3) * PER_LO + MX) : "memory");
        } else
          asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      }
      if (kt + S - 1 < kt1) issue(kt + S - 1, (it + S - 1) % S);
      if (kt + 1 < kt1) read_codes((it + 1) % S, kt + 1);
      const uint8_t* As_ = lds + slot * STAGE;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        half8_t af[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int r = i * 16 + l16, ch = 2 * g4 + ks;
          af[i] = *reinterpret_cast<const half8_t*>(As_ + r * 128 + ((ch ^ (r & 7)) * 16));
          __builtin_amdgcn_sched_barrier(0);  // issue in use order
        }
        // (past the last step the rebuilds fill an unused buffer: a runtime
        // condition here would split the MFMA chain)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          mfma4_rebuild_ab(acc[2 * p][0], acc[2 * p][1], acc[2 * p + 1][0], acc[2 * p + 1][1], af[2 * p], af[2 * p],
                           af[2 * p + 1], af[2 * p + 1], bcur[ks][0], bcur[ks][1], bcur[ks][0], bcur[ks][1],
                           ks ? cw[p].y : cw[p].x, cm[p], bnxt[ks][p]);
#pragma unroll
        for (int i = 4; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) mfma16x16x32_acc_ordered(acc[i][j], af[i], bcur[ks][j]);
      }
    };
    // groups of steps: every split has a multiple of 4 steps (META4) or an
    // even number (the host guarantees it), so the MFMA chain is one piece
    // of code
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    if constexpr (META4) {
      for (int kt = kt0; kt < kt1; kt += 4) {
        step(I0{}, kt, bA, bB);
        step(I1{}, kt + 1, bB, bA);
        step(I2{}, kt + 2, bA, bB);
        step(I3{}, kt + 3, bB, bA);
      }
    } else {
      for (int kt = kt0; kt < kt1; kt += 2) {
        step(I0{}, kt, bA, bB);
        step(I1{}, kt + 1, bB, bA);
      }
    }
    // the last MFMAs' results are read by VALU instructions below
    mfma_results_ready();
  }

#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n_blk + wave * 32 + j * 16 + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m_base + i * 16 + 4 * g4 + r;
        if (m < M && n < N) {
          if (partial)
            partial[((int64_t)blockIdx.y * M + m) * N + n] = acc[i][j][r];
          else
            epilogue_store(epi, m, n, acc[i][j][r]);
        }
      }
    }
  }
}

// The decode GEMM with the prefill kernel's arrangement: 4 waves side by
// side in N (64 weight rows each, one wave per SIMD) over the batch's 16 MB
// rows, K step 64, each A fragment feeding 4 MFMAs; the same copies as the
// prefill kernel (scalar base + 32-bit lane offsets, unconditional, {min,
// scale} 4 steps at a time); K is split over ranges of a multiple of 4
// steps, either per tile (SK false: grid.y splits) or as a stream-K schedule
// (SK true: one block per CU, each an equal run of (tile, step) units).
// Slot = 16-row block of one k slice (2 MB slots per step): copies in slots
// 0..7; the 8 rebuilds of the next step's weights (13 instructions each) in
// halves over the last 16 slots when there are 16 or more (MB >= 8), else
// whole, one with each group of 4 MFMAs, in the last 8 slots.
// Slice ks gives lane group g the k chunk 2 g + ks (8 values), as the
// two-waves-per-SIMD decode kernel does, so under the same split the two add
// the same products in the same order (outputs identical bit for bit).
template <int MB, bool SK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_decode_w4_kernel(
    const uint16_t* __restrict__ A, int64_t M, int64_t lda, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ meta, int64_t N, int64_t K, int k_tiles_per_split, int sk_per, Epilogue epi,
    float* __restrict__ partial) {
  constexpr int ROWS = MB * 16, NSL = 2 * MB;        // A rows per block, row-block slots per step
  constexpr int NQ = ROWS / 8;                       // A copies per step (8 rows of 128 B)
  constexpr int A_MAX = (NQ + 3) / 4, EXTRA = NQ % 4 ? NQ % 4 : 4;  // waves below EXTRA issue A_MAX, others one fewer
  constexpr int A_BYTES = ROWS * 128, C_BYTES = 256 * 32, M_BYTES = 256 * 16;
  constexpr int SC = 3, FN = 4, TN = 64;
  constexpr int RING = NSL % 4 == 0 ? 4 : 6;         // A fragment ring (divides NSL), read 3 slots ahead
  static_assert(NSL % RING == 0 && NSL >= 8, "slot layout");
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds0[A_BYTES], a_lds1[A_BYTES], a_lds2[A_BYTES],
      a_lds3[A_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t c_lds[SC * C_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t m_lds[2 * M_BYTES];
  auto a_st = [&](auto s) -> uint8_t* {
    constexpr int S = decltype(s)::value;
    return S == 0 ? a_lds0 : S == 1 ? a_lds1 : S == 2 ? a_lds2 : a_lds3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave, fr = lane & 15, fk = lane >> 4;
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  const int64_t m0 = (int64_t)blockIdx.z * ROWS;
  const int KT = (int)(K / BK);
  // One segment: K steps kt0..kt1 (a positive multiple of 4, host) of the
  // 256-column tile at n0; fp32 partials, if any, to slab `slab`.
  auto segment = [&](const int64_t n0, const int kt0, const int kt1, const int slab) {

    const uint8_t* a_blk = reinterpret_cast<const uint8_t*>(A + m0 * lda);
    const uint8_t* c_blk = codes + n0 * (K / 2);
    const uint8_t* m_blk = reinterpret_cast<const uint8_t*>(meta + n0 * (K / 64) * 2);
    // A: instruction q = w + 4t (q < NQ) fills rows 8q..8q+7; codes: instruction
    // p = w, w + 4 fills rows 32p..32p+31; meta: wave w rows 64w..64w+63
    uint32_t a_off[A_MAX], c_off[2];
#pragma unroll
    for (int t = 0; t < A_MAX; ++t) {
      const int r = 8 * (wave + 4 * t) + (lane >> 3);
      a_off[t] = (uint32_t)((min(m0 + r, M - 1) - m0) * lda * 2 + ((lane & 7) ^ (r & 7)) * 16);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
      c_off[t] = (uint32_t)((min(n0 + 32 * (wave + 4 * t) + (lane >> 1), N - 1) - n0) * (K / 2) + (lane & 1) * 16);
    const uint32_t m_off = (uint32_t)((min(n0 + 64 * wave + lane, N - 1) - n0) * (K / 64) * 4);
    const uint32_t c_base = (uint32_t)(uintptr_t)c_lds, m_base = (uint32_t)(uintptr_t)m_lds;
    auto issue_a = [&](auto s, int kt) {
      const uint32_t dst = (uint32_t)(uintptr_t)a_st(s) + swave * 1024;
#pragma unroll
      for (int t = 0; t < A_MAX; ++t)
        if (t + 1 < A_MAX || swave < EXTRA) dma_lds16_s(a_off[t], a_blk + (int64_t)kt * 128, dst + t * 4096);
    };
    auto issue_codes = [&](int kt) {
      const uint32_t dst = c_base + (kt % SC) * C_BYTES;
#pragma unroll
      for (int t = 0; t < 2; ++t) dma_lds16_s(c_off[t], c_blk + (int64_t)kt * 32, dst + (swave + 4 * t) * 1024);
    };
    // {min, scale} of 4-step group g into buffer buf
    auto issue_meta = [&](int g, int buf) {
      dma_lds16_s(m_off, m_blk + (int64_t)g * 16, m_base + buf * M_BYTES + swave * 1024);
    };
    uint32_t cw[2][FN], cm[FN];
    auto read_codes = [&](int kt) {
      const uint8_t* slot = c_lds + (kt % SC) * C_BYTES;
      const uint8_t* mrow = m_lds + ((kt >> 2) & 1) * M_BYTES + (kt & 3) * 4;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * TN + j * 16 + fr;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) cw[ks][j] = *reinterpret_cast<const uint32_t*>(slot + row * 32 + (2 * fk + ks) * 4);
        cm[j] = *reinterpret_cast<const uint32_t*>(mrow + row * 16);
      }
    };
    auto rebuild = [&](int ks, int j) {
      const half_t mn = __builtin_bit_cast(half_t, (uint16_t)(cm[j] & 0xFFFF));
      const half_t sc = __builtin_bit_cast(half_t, (uint16_t)(cm[j] >> 16));
      const half2_t mn2 = {mn, mn}, s2 = {sc, sc};
      uint32_t o[4];
      dequant8(cw[ks][j], mn2, s2, o);
      return __builtin_bit_cast(half8_t, make_uint4(o[0], o[1], o[2], o[3]));
    };
    auto a_frag = [&](const uint8_t* As_, int ks, int i) {
      const int r = i * 16 + fr;
      return *reinterpret_cast<const half8_t*>(As_ + r * 128 + (((2 * fk + ks) ^ (r & 7)) * 16));
    };

    float4_t acc[MB][FN];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};

    // prologue: codes and A of the split's first three steps, {min, scale} of
    // its first 4-step group; operand of the first step rebuilt
    issue_codes(kt0);
    issue_codes(kt0 + 1);
    issue_codes(kt0 + 2);
    issue_meta(kt0 >> 2, (kt0 >> 2) & 1);
    issue_a(I0{}, kt0);
    issue_a(I1{}, kt0 + 1);
    issue_a(I2{}, kt0 + 2);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    half8_t bA[2][FN], bB[2][FN];
    read_codes(kt0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < FN; ++j) bA[ks][j] = rebuild(ks, j);
    half8_t fa[RING];
#pragma unroll
    for (int t = 0; t < 3; ++t) fa[t] = a_frag(a_lds0, t / MB, t % MB);

    // step kt (S = (kt - kt0) % 4): as in the prefill kernel; per wave A_w + 2
    // copies, + 1 {min, scale} copy when S == 0 (group kt/4 + 1)
    auto step = [&](auto s, int kt) {
      constexpr int S = decltype(s)::value;
      constexpr int P = S & 1;
      using S3 = std::integral_constant<int, (S + 3) % 4>;
      using S1 = std::integral_constant<int, (S + 1) % 4>;
      half8_t(&bcur)[2][FN] = P == 0 ? bA : bB;
      half8_t(&bnxt)[2][FN] = P == 0 ? bB : bA;
      const uint8_t* As_ = a_st(s);
      read_codes(kt + 1);  // stale but harmless past the split's last step
      const int kc = min(kt + 3, kt1 - 1);
      const uint8_t* a_step = a_blk + (int64_t)kc * 128;
      const uint8_t* c_step = c_blk + (int64_t)kc * 32;
      const uint32_t a_dst = (uint32_t)(uintptr_t)a_st(S3{}) + swave * 1024;
      const uint32_t c_dst = c_base + ((kt + 3) % SC) * C_BYTES;
      const int gm = min((kt >> 2) + 1, (kt1 >> 2) - 1);
      uint32_t hp0 = 0, hp1 = 0, ho0 = 0;  // a rebuild between its two halves
      static_for<NSL>([&](auto sc) {
        constexpr int SL = decltype(sc)::value;
        constexpr int ks = SL / MB, i = SL % MB;
        if constexpr (SL < A_MAX) {
          if (SL + 1 < A_MAX || swave < EXTRA) dma_lds16_s(a_off[SL], a_step, a_dst + SL * 4096);
        } else if constexpr (SL == 5 || SL == 6) {
          dma_lds16_s(c_off[SL - 5], c_step, c_dst + (swave + 4 * (SL - 5)) * 1024);
        } else if constexpr (SL == 7 && S == 0) {
          // group kt/4 + 1 into its buffer; past the split's end the copy is
          // clamped to the last group but still lands in the buffer no later
          // step reads
          issue_meta(gm, ((kt >> 2) + 1) & 1);
        }
        constexpr int NX = SL + 3;
        fa[NX % RING] = NX < NSL ? a_frag(As_, NX / MB, NX % MB) : a_frag(a_st(S1{}), (NX - NSL) / MB, (NX - NSL) % MB);
        __builtin_amdgcn_sched_barrier(0);
        const half8_t& af = fa[SL % RING];
        if constexpr (NSL >= 16 && SL >= NSL - 16) {
          // 16 or more slots: each rebuild in two halves over two slots (at
          // most 7 VALU instructions beside each group of 4 MFMAs)
          constexpr int q = SL - (NSL - 16), r = q / 2;
          if constexpr (q % 2 == 0) {
            mfma4_rebuild_h1(acc[i][0], acc[i][1], acc[i][2], acc[i][3], af, bcur[ks][0], bcur[ks][1], bcur[ks][2],
                             bcur[ks][3], cw[r / FN][r % FN], hp0, hp1, ho0);
          } else {
            half8_t nb;
            mfma4_rebuild_h2(acc[i][0], acc[i][1], acc[i][2], acc[i][3], af, bcur[ks][0], bcur[ks][1], bcur[ks][2],
                             bcur[ks][3], hp0, hp1, ho0, cm[r % FN], nb);
            bnxt[r / FN][r % FN] = nb;
          }
        } else if constexpr (NSL < 16 && SL >= NSL - 8) {
          constexpr int r = SL - (NSL - 8);
          half8_t nb;
          mfma4_rebuild_ab(acc[i][0], acc[i][1], acc[i][2], acc[i][3], af, af, af, af, bcur[ks][0], bcur[ks][1],
                           bcur[ks][2], bcur[ks][3], cw[r / FN][r % FN], cm[r % FN], nb);
          bnxt[r / FN][r % FN] = nb;
        } else {
#pragma unroll
          for (int j = 0; j < FN; ++j) mfma16x16x32_acc_ordered(acc[i][j], af, bcur[ks][j]);
        }
      });
      if (swave < EXTRA) {
        if constexpr (S == 0)
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(A_MAX + 3) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(A_MAX + 2) : "memory");
      } else {
        if constexpr (S == 0)
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(A_MAX + 2) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(A_MAX + 1) : "memory");
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), where the compiler sees it
    };
    for (int kt = kt0; kt < kt1; kt += 4) {
      step(I0{}, kt);
      step(I1{}, kt + 1);
      step(I2{}, kt + 2);
      step(I3{}, kt + 3);
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    mfma_results_ready();  // the last MFMAs' results are read below

    if (SK || partial) {
      // fp32 split-K partials: one element per store, 16 consecutive columns
      // per 16 lanes (staging them through LDS first was slower here)
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t n = n0 + wn * TN + j * 16 + fr;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + i * 16 + 4 * fk + r;
            if (m < M && n < N) partial[((int64_t)slab * M + m) * N + n] = acc[i][j][r];
          }
        }
      return;
    }
    // Final outputs: staged through LDS (the code slots, free now), 16 rows x 64
    // columns per wave at a time (row stride 68 floats), so that each lane
    // holds 16 consecutive columns of one row and runs the epilogue on 8-column
    // chunks (16-byte loads of bias and residual, 16-byte stores) instead of one
    // element at a time.
    {
      constexpr int SROW = 68;
      static_assert(4 * 16 * SROW * 4 <= SC * C_BYTES, "epilogue staging fits the code slots");
      float* stg = reinterpret_cast<float*>(c_lds) + wn * (16 * SROW);
      const bool vec = epilogue_vec_ok(epi);
      const int rr = lane >> 2, cs = (lane & 3) * 16;
      static_for<MB>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) stg[(4 * fk + r) * SROW + j * 16 + fr] = acc[i][j][r];
        __syncthreads();
        const int64_t m = m0 + i * 16 + rr;
        const int64_t nw = n0 + wn * TN + cs;  // this lane's 16 columns
        const float* src = stg + rr * SROW + cs;
        if (m < M) {
#pragma unroll
          for (int c = 0; c < 16; c += 8) {
            const float4 lo = *reinterpret_cast<const float4*>(src + c);
            const float4 hi = *reinterpret_cast<const float4*>(src + c + 4);
            const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            epilogue_store8(epi, m, nw + c, v, N, vec);
          }
        }
        __syncthreads();
      });
    }
  };
  if constexpr (SK) {
    // Stream K (one block per CU): the block runs (256-column tile, K step)
    // units blockIdx.x * sk_per onward, sk_per of them, tile-major, in one
    // segment per tile it touches; a tile's segments go to partial slabs 0,
    // 1, ... in the order of the blocks that run them.  A segment's LDS reads
    // all complete before its last barrier, so the next segment's copies may
    // overwrite the rings.  (32-bit unit arithmetic: the host keeps
    // n_tiles * KT below 2^31.)
    const int n_tiles = (int)((N + 255) / 256);
    int unit = (int)blockIdx.x * sk_per;
    const int unit_end = min(unit + sk_per, n_tiles * KT);
    while (unit < unit_end) {
      const int tile = unit / KT;
      const int kt0 = unit - tile * KT;
      const int kt1 = min(KT, kt0 + (unit_end - unit));
      segment((int64_t)tile * 256, kt0, kt1, (int)blockIdx.x - tile * KT / sk_per);
      unit = tile * KT + kt1;
    }
  } else {
    // Split K: tile blockIdx.x, steps from blockIdx.y * k_tiles_per_split,
    // partial slab blockIdx.y (no partials when K is not split)
    const int kt0 = blockIdx.y * k_tiles_per_split;
    segment((int64_t)blockIdx.x * 256, kt0, min(KT, kt0 + k_tiles_per_split), (int)blockIdx.y);
  }
}

// Sum of the split-K partials ([split][M][N] fp32), in split order from
// zero, then the epilogue: 8 columns of one row per thread, with 16-byte
// loads when N is a multiple of 8 (every chunk whole and aligned).  With
// sk_per > 0 (the stream-K schedule of the decode kernel over KT steps) the
// 256-column tile t holds one slab per block that ran part of it:
// (t + 1) KT / sk_per - t KT / sk_per of them, rounded as the kernel splits.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial, int splits, int64_t M,
                                                            int64_t N, Epilogue epi, int64_t KT = 0, int sk_per = 0) {
  const int64_t nc = (N + 7) / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= M * nc) return;
  const int64_t m = t / nc, n = (t - m * nc) * 8;
  const int64_t mn = M * N;
  if (sk_per > 0) {
    const int64_t tile = n / 256;
    splits = (int)(((tile + 1) * KT - 1) / sk_per - tile * KT / sk_per + 1);
  }
  const float* p = partial + m * N + n;
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = 0.f;
  if (N % 8 == 0) {
    for (int z = 0; z < splits; ++z) {
      const float4 a = *reinterpret_cast<const float4*>(p + z * mn);
      const float4 b = *reinterpret_cast<const float4*>(p + z * mn + 4);
      v[0] += a.x, v[1] += a.y, v[2] += a.z, v[3] += a.w;
      v[4] += b.x, v[5] += b.y, v[6] += b.z, v[7] += b.w;
    }
  } else {
    for (int z = 0; z < splits; ++z)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (n + k < N) v[k] += p[z * mn + k];
  }
  epilogue_store8(epi, m, n, v, N, epilogue_vec_ok(epi));
}

// Blocks of splitk_reduce_kernel for an M x N output.
inline unsigned reduce_blocks(int64_t M, int64_t N) { return (unsigned)ceil_div(M * ((N + 7) / 8), 256); }

// Split-K workspace, grown on demand and kept for the life of the process.
struct Workspace {
  float* ptr = nullptr;
  size_t bytes = 0;
  int device = -1;
};
thread_local Workspace g_ws;

// While fq_dequant_gemm_noalloc runs on this thread: the fixed buffer its
// partials go to (nothing is allocated).
struct FixedWorkspace {
  float* ptr;
  size_t bytes;
};
thread_local const FixedWorkspace* g_fixed_ws = nullptr;

fq_status get_workspace(size_t bytes, float** out) {
  if (g_fixed_ws) {
    if (bytes > g_fixed_ws->bytes)
      return fail(FQ_ERR_INVALID, "fq_dequant_gemm_noalloc: this shape needs " + std::to_string(bytes) +
                                      " bytes of split-K partials, more than the " +
                                      std::to_string(g_fixed_ws->bytes) + "-byte scratch");
    *out = g_fixed_ws->ptr;
    return FQ_OK;
  }
  int dev = 0;
  FQ_HIP(hipGetDevice(&dev));
  if (g_ws.ptr && (g_ws.bytes < bytes || g_ws.device != dev)) {
    FQ_HIP(hipDeviceSynchronize());
    (void)hipFree(g_ws.ptr);
    g_ws.ptr = nullptr;
    g_ws.bytes = 0;
  }
  if (!g_ws.ptr) {
    hipError_t e = hipMalloc(&g_ws.ptr, bytes);
    if (e != hipSuccess) {
      g_ws.ptr = nullptr;
      return fail(FQ_ERR_OOM, "fq_dequant_gemm: split-K workspace allocation failed");
    }
    g_ws.bytes = bytes;
    g_ws.device = dev;
  }
  *out = g_ws.ptr;
  return FQ_OK;
}

template <int MB>
fq_status run_skinny(const uint16_t* A, int64_t M, int64_t lda, const fq_weight* W, const Epilogue& epi, hipStream_t st) {
  const int64_t N = W->n;
  const int KT = (int)(W->k / BK);
  const int64_t nblk = ceil_div(N, 256) * ceil_div(M, 16 * MB);
  // aim for ~2 blocks per CU, each split at least 4 K steps long
  int splits = (int)std::max<int64_t>(1, std::min<int64_t>(KT / 4, ceil_div(512, nblk)));
  const int kps = (KT + splits - 1) / splits;
  splits = (KT + kps - 1) / kps;
  float* partial = nullptr;
  if (splits > 1) FQ_TRY(get_workspace((size_t)splits * M * N * sizeof(float), &partial));
  const dim3 grid((unsigned)ceil_div(N, 256), (unsigned)splits, (unsigned)ceil_div(M, 16 * MB));
  if (W->kind == FQ_WEIGHT_PACKED4)
    gemm_skinny_kernel<MB, true><<<grid, dim3(256), 0, st>>>(A, M, lda, W->packed.codes, W->packed.meta, nullptr, N,
                                                             W->k, kps, epi, partial);
  else
    gemm_skinny_kernel<MB, false><<<grid, dim3(256), 0, st>>>(A, M, lda, nullptr, nullptr, W->w16, N, W->k, kps, epi,
                                                              partial);
  FQ_TRY(launch_check("gemm_skinny_kernel"));
  if (splits > 1) {
    splitk_reduce_kernel<<<dim3(reduce_blocks(M, N)), dim3(256), 0, st>>>(partial, splits, M, N, epi);
    FQ_TRY(launch_check("splitk_reduce_kernel"));
  }
  return FQ_OK;
}

// Split count for the 4-bit decode GEMM: blocks run one per CU (the LDS ring
// takes most of a CU's LDS), so pick the split that minimises rounds of 256
// blocks x (K steps per block + ring fill), plus the fp32 partial traffic
// (written and read back by the reduction) priced at 4 TB/s.
int decode_splits(int64_t nblk, int KT, int64_t M, int64_t N, int MB, double* t_out) {
  // measured: one K step of a block takes ~1.3 us at 9 row groups
  const double step_us = std::max(0.15, 0.145 * MB);
  int best = 1;
  double best_t = 1e30;
  for (int s = 1; s <= std::min(16, std::max(1, KT / 4)); ++s) {
    const int kps = (KT + s - 1) / s;
    const int splits = (KT + kps - 1) / kps;
    const double rounds = (double)ceil_div(nblk * splits, 256);
    const double t = rounds * (kps + 6) * step_us + (splits > 1 ? splits * (double)M * N * 8.0 / 4e6 : 0.0);
    if (t < best_t - 1e-9) {
      best_t = t;
      best = s;
    }
  }
  *t_out = best_t;
  return best;
}

// Stream-K schedule of the one-wave-per-SIMD decode kernel: 256 / zb blocks
// per row group (one per CU), each running `per` consecutive (256-column tile,
// K step) units, a multiple of 4, in one segment per tile it touches; each
// segment writes an fp32 partial slab that the reduction sums in block order.
// It removes the partly filled last round of a split-K grid at the price of a
// ring fill per segment and more partial slabs.  Priced with the split-K
// model: steps plus ring fills of the busiest block, partials at 4 TB/s.
struct StreamK {
  int per = 0;        // units per block
  int blocks = 0;     // blocks per row group
  int max_slabs = 0;  // the most segments any tile has
  double t = 1e30;    // predicted time, us
};
StreamK stream_k_plan(int64_t n_tiles, int KT, int64_t zb, int64_t M, int MB) {
  const double step_us = std::max(0.15, 0.145 * MB);
  StreamK p;
  const int64_t total = n_tiles * KT;
  const int64_t per = (ceil_div(total, std::max<int64_t>(1, 256 / zb)) + 3) & ~int64_t{3};
  int64_t segs = 0, max_s = 0;
  for (int64_t t = 0; t < n_tiles; ++t) {
    const int64_t sgs = ((t + 1) * KT - 1) / per - t * KT / per + 1;
    segs += sgs;
    max_s = std::max(max_s, sgs);
  }
  p.per = (int)per;
  p.blocks = (int)ceil_div(total, per);
  p.max_slabs = (int)max_s;
  p.t = (per + 6.0 * (double)std::min<int64_t>(ceil_div(per, KT) + 1, n_tiles)) * step_us +
        (double)segs * M * 256 * 8.0 / 4e6;
  return p;
}

template <int MB>
fq_status run_decode(const uint16_t* A, int64_t M, int64_t lda, const fq_weight* W, const Epilogue& epi,
                     hipStream_t st) {
  const int64_t N = W->n;
  const int KT = (int)(W->k / BK);
  const int64_t zb = ceil_div(M, 16 * MB), n_tiles = ceil_div(N, 256);
  double split_t = 0.0;
  int splits = decode_splits(n_tiles * zb, KT, M, N, MB, &split_t);
  // the kernel runs K steps in groups: a multiple of 4 per split when the
  // {min, scale} go 4 steps at a time (K a multiple of 256 and that array
  // 16-byte aligned), else an even number (KT is even here)
  const bool meta4 = KT % 4 == 0 && (uintptr_t)W->packed.meta % 16 == 0;
  const int kps = meta4 ? ((KT + splits - 1) / splits + 3) & ~3 : ((KT + splits - 1) / splits + 1) & ~1;
  splits = (KT + kps - 1) / kps;
  // stream K instead where every block gets at least 16 steps and the model
  // predicts 5 % less time (one-wave-per-SIMD kernel only)
  const StreamK sk = meta4 ? stream_k_plan(n_tiles, KT, zb, M, MB) : StreamK{};
  if (sk.per >= 16 && sk.t < 0.95 * split_t && n_tiles * KT < (int64_t{1} << 31)) {
    float* partial = nullptr;
    FQ_TRY(get_workspace((size_t)sk.max_slabs * M * N * sizeof(float), &partial));
    gemm_decode_w4_kernel<MB, true><<<dim3((unsigned)sk.blocks, 1, (unsigned)zb), dim3(256), 0, st>>>(
        A, M, lda, W->packed.codes, W->packed.meta, N, W->k, 0, sk.per, epi, partial);
    FQ_TRY(launch_check("gemm_decode_w4_kernel"));
    splitk_reduce_kernel<<<dim3(reduce_blocks(M, N)), dim3(256), 0, st>>>(partial, 0, M, N, epi, KT, sk.per);
    return launch_check("splitk_reduce_kernel");
  }
  float* partial = nullptr;
  if (splits > 1) FQ_TRY(get_workspace((size_t)splits * M * N * sizeof(float), &partial));
  const dim3 grid((unsigned)n_tiles, (unsigned)splits, (unsigned)zb);
  // one wave per SIMD when the {min, scale} go 4 steps at a time, else the
  // two-waves-per-SIMD kernel
  if (meta4) {
    gemm_decode_w4_kernel<MB, false><<<grid, dim3(256), 0, st>>>(A, M, lda, W->packed.codes, W->packed.meta, N, W->k,
                                                                 kps, 0, epi, partial);
    FQ_TRY(launch_check("gemm_decode_w4_kernel"));
  } else {
    gemm_decode8_kernel<MB, false><<<grid, dim3(512), 0, st>>>(A, M, lda, W->packed.codes, W->packed.meta, N, W->k,
                                                               kps, epi, partial);
    FQ_TRY(launch_check("gemm_decode8_kernel"));
  }
  if (splits > 1) {
    splitk_reduce_kernel<<<dim3(reduce_blocks(M, N)), dim3(256), 0, st>>>(partial, splits, M, N, epi);
    FQ_TRY(launch_check("splitk_reduce_kernel"));
  }
  return FQ_OK;
}

fq_status dispatch_skinny(const uint16_t* A, int64_t M, int64_t lda, const fq_weight* W, const Epilogue& epi,
                          hipStream_t st) {
  const int64_t mb = ceil_div(M, 16);
  // the streaming decode kernel for 4-bit weights and even K steps (and lda
  // and K small enough for its 32-bit per-lane copy offsets); below 49 rows
  // it runs with 4 row blocks (the rows past M are clamped reads, never
  // stored): the weight stream, not the MFMAs, sets its time there
  if (W->kind == FQ_WEIGHT_PACKED4 && (W->k / BK) % 2 == 0 && lda <= (int64_t{1} << 22) && W->k <= (int64_t{1} << 24)) {
    if (mb <= 4) return run_decode<4>(A, M, lda, W, epi, st);
    if (mb <= 6) return run_decode<6>(A, M, lda, W, epi, st);
    if (mb <= 8) return run_decode<8>(A, M, lda, W, epi, st);
    if (mb <= 9) return run_decode<9>(A, M, lda, W, epi, st);
    return run_decode<8>(A, M, lda, W, epi, st);  // 129..256 rows: two row groups of 128
  }
  if (mb <= 1) return run_skinny<1>(A, M, lda, W, epi, st);
  if (mb <= 2) return run_skinny<2>(A, M, lda, W, epi, st);
  if (mb <= 3) return run_skinny<3>(A, M, lda, W, epi, st);
  if (mb <= 4) return run_skinny<4>(A, M, lda, W, epi, st);
  if (mb <= 6) return run_skinny<6>(A, M, lda, W, epi, st);
  if (mb <= 8) return run_skinny<8>(A, M, lda, W, epi, st);
  if (mb <= 9) return run_skinny<9>(A, M, lda, W, epi, st);
  return run_skinny<8>(A, M, lda, W, epi, st);  // 129..256 rows: two row groups of 128
}

template <int BM, int BN, int WM, int WN>
fq_status run_gemm(const uint16_t* A, int64_t M, int64_t lda, const fq_weight* W, const Epilogue& epi, int splits,
                   hipStream_t st) {
  const int64_t tiles = ceil_div(M, BM) * ceil_div(W->n, BN);
  const int KT = (int)(W->k / BK);
  splits = std::max(1, std::min(splits, KT));
  const int kps = (KT + splits - 1) / splits;
  splits = (KT + kps - 1) / kps;
  float* partial = nullptr;
  if (splits > 1) FQ_TRY(get_workspace((size_t)splits * M * W->n * sizeof(float), &partial));
  const dim3 grid((unsigned)tiles, 1, (unsigned)splits);
  const dim3 block(WM * WN * 64);
  if (W->kind == FQ_WEIGHT_PACKED4)
    gemm_kernel<BM, BN, WM, WN, true><<<grid, block, 0, st>>>(A, M, lda, W->packed.codes, W->packed.meta, nullptr,
                                                              W->n, W->k, kps, epi, partial);
  else
    gemm_kernel<BM, BN, WM, WN, false><<<grid, block, 0, st>>>(A, M, lda, nullptr, nullptr, W->w16, W->n, W->k, kps,
                                                               epi, partial);
  FQ_TRY(launch_check("gemm_kernel"));
  if (splits > 1) {
    splitk_reduce_kernel<<<dim3(reduce_blocks(M, W->n)), dim3(256), 0, st>>>(partial, splits, M, W->n, epi);
    FQ_TRY(launch_check("splitk_reduce_kernel"));
  }
  return FQ_OK;
}

}  // namespace
}  // namespace fq

using namespace fq;

// Shapes the 256 x 256 one-wave-per-SIMD kernel takes: packed weights, enough
// tiles to fill the chip, K a multiple of 256 (its K loop), 32-bit per-lane
// copy offsets that cannot overflow (up to 255 rows of lda or K / 2 bytes past
// the block's first row) and a 16-byte aligned {min, scale} array (copied 16
// bytes per row).
static bool tile256_fits(int64_t M, int64_t N, int64_t K, int64_t lda, const fq_weight* W) {
  return M >= 1024 && N >= 1024 && ceil_div(M, 256) * ceil_div(N, 256) >= 128 && W->kind == FQ_WEIGHT_PACKED4 &&
         K % 256 == 0 && lda <= (int64_t{1} << 22) && K <= (int64_t{1} << 24) &&
         (uintptr_t)W->packed.meta % 16 == 0;
}


// The projection GEMM behind both entry points; `timed`: record the launch
// for fq_timing_* (event creation allocates, so the allocation-free entry
// point never records).
static fq_status dequant_gemm(const uint16_t* A, int64_t M, int64_t lda, const fq_weight* W, const uint16_t* bias,
                              const uint16_t* residual, int64_t ldr, uint32_t epilogue, float qscale,
                              int64_t qscale_cols, void* C, int64_t ldc, void* stream, bool timed) {
  FQ_CHECK_ARG(W != nullptr, "fq_dequant_gemm: W is NULL");
  FQ_CHECK_ARG(W->kind == FQ_WEIGHT_PACKED4 || W->kind == FQ_WEIGHT_F16, "fq_dequant_gemm: unknown weight kind");
  const int64_t N = W->n, K = W->k;
  FQ_CHECK_ARG(M >= 0 && N > 0 && K > 0, "fq_dequant_gemm: bad shape");
  FQ_CHECK_ARG(K % 64 == 0, "fq_dequant_gemm: K must be a multiple of 64");
  FQ_CHECK_ARG(lda >= K && lda % 8 == 0, "fq_dequant_gemm: lda must be >= K and a multiple of 8");
  FQ_CHECK_ARG(ldc >= N, "fq_dequant_gemm: ldc < N");
  if (W->kind == FQ_WEIGHT_PACKED4) {
    if (W->packed.group != FQ_GROUP) return fail(FQ_ERR_UNSUPPORTED, "fq_dequant_gemm: only group 64 is implemented");
    FQ_CHECK_ARG(W->packed.rows == N && W->packed.cols == K, "fq_dequant_gemm: packed shape differs from n/k");
    FQ_CHECK_ARG(W->packed.codes && W->packed.meta, "fq_dequant_gemm: NULL packed weight");
    FQ_CHECK_ARG(((uintptr_t)W->packed.codes % 16 == 0) && ((uintptr_t)W->packed.meta % 4 == 0),
                 "fq_dequant_gemm: packed weight must be 16-byte aligned");
  } else {
    FQ_CHECK_ARG(W->w16 != nullptr && (uintptr_t)W->w16 % 16 == 0, "fq_dequant_gemm: fp16 weight NULL or misaligned");
  }
  FQ_CHECK_ARG(!(epilogue & FQ_EPI_BIAS) || bias, "fq_dequant_gemm: BIAS without bias");
  FQ_CHECK_ARG(!(epilogue & FQ_EPI_RESIDUAL) || (residual && ldr >= N), "fq_dequant_gemm: RESIDUAL without residual");
  if (M == 0) return FQ_OK;
  FQ_CHECK_ARG(A && C, "fq_dequant_gemm: NULL A or C");
  FQ_CHECK_ARG((uintptr_t)A % 16 == 0, "fq_dequant_gemm: A must be 16-byte aligned");
  Epilogue epi{bias, residual, ldr, epilogue, qscale, qscale_cols, C, ldc};
  hipStream_t st = as_stream(stream);
  // Tile choice: enough tiles to fill 256 CUs, split-K when the grid is small.
  const int KT = (int)(K / 64);
  const int cls = (epilogue & FQ_EPI_F32OUT) ? FQ_KC_LM_HEAD : (M > 256 ? FQ_KC_GEMM_PREFILL : FQ_KC_GEMM_DECODE);
  const int tk = timed ? timing_begin(cls, st) : -1;
  fq_status r;
  if (M <= 256) {
    r = dispatch_skinny(A, M, lda, W, epi, st);
  } else if (tile256_fits(M, N, K, lda, W)) {
    const dim3 grid((unsigned)(ceil_div(M, 256) * ceil_div(N, 256)));
    gemm_w4_kernel<false><<<grid, dim3(256), 0, st>>>(A, M, lda, W->packed.codes, W->packed.meta, N, K, epi,
                                                      KvAppend{});
    r = launch_check("gemm_w4_kernel");
  } else if (M >= 1024 && N >= 1024 && ceil_div(M, 256) * ceil_div(N, 128) >= 256) {
    const dim3 grid((unsigned)(ceil_div(M, 256) * ceil_div(N, 128)));
    if (W->kind == FQ_WEIGHT_PACKED4)
      gemm_big_kernel<true><<<grid, dim3(256), 0, st>>>(A, M, lda, W->packed.codes, W->packed.meta, nullptr, N, K, epi);
    else
      gemm_big_kernel<false><<<grid, dim3(256), 0, st>>>(A, M, lda, nullptr, nullptr, W->w16, N, K, epi);
    r = launch_check("gemm_big_kernel");
  } else {
    const int64_t tiles = ceil_div(M, 128) * ceil_div(N, 128);
    const int splits = tiles >= 256 ? 1 : (int)std::max<int64_t>(1, std::min<int64_t>(KT / 4, 512 / tiles));
    r = run_gemm<128, 128, 2, 2>(A, M, lda, W, epi, splits, st);
  }
  if (r == FQ_OK && tk >= 0) {
    const double wbytes = W->kind == FQ_WEIGHT_PACKED4 ? 0.5625 * N * K : 2.0 * N * K;
    const double cbytes = (epilogue & FQ_EPI_F32OUT) ? 4.0 * M * N : 2.0 * M * N;
    const double bytes = 2.0 * M * K + wbytes + cbytes + ((epilogue & FQ_EPI_RESIDUAL) ? 2.0 * M * N : 0.0) +
                         ((epilogue & FQ_EPI_BIAS) ? 2.0 * N : 0.0);
    timing_end(tk, cls, 2.0 * M * N * K, bytes, st);
  }
  return r;
}

extern "C" fq_status fq_dequant_gemm(const uint16_t* A, int64_t M, int64_t lda, const fq_weight* W,
                                     const uint16_t* bias, const uint16_t* residual, int64_t ldr, uint32_t epilogue,
                                     float qscale, int64_t qscale_cols, void* C, int64_t ldc, void* stream) {
  clear_error();
  return dequant_gemm(A, M, lda, W, bias, residual, ldr, epilogue, qscale, qscale_cols, C, ldc, stream, true);
}

// ---- allocation-free projection GEMM ---------------------------------------
// The split-K partials of fq_dequant_gemm_noalloc live in this array, one copy
// per GPU (kept until the process ends).  Host code never uses its name as an
// address: the device address of each GPU's copy is looked up once per device
// (hipGetSymbolAddress, with that device current) and that pointer is what
// the kernels receive.
constexpr size_t kScratchBytes = size_t{64} << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

fq_status scratch_for_current_device(float** out) {
  int dev = 0;
  FQ_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(FQ_ERR_UNSUPPORTED, "fq_dequant_gemm_noalloc: device index too large");
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "fq_dequant_gemm_noalloc: hipGetSymbolAddress");
    }
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return FQ_OK;
}

// Points get_workspace at the scratch for the duration of one call.
struct FixedWorkspaceScope {
  FixedWorkspace ws;
  explicit FixedWorkspaceScope(float* p) : ws{p, kScratchBytes} { g_fixed_ws = &ws; }
  ~FixedWorkspaceScope() { g_fixed_ws = nullptr; }
};
}  // namespace

extern "C" fq_status fq_dequant_gemm_noalloc(const uint16_t* A, int64_t M, int64_t lda, const fq_weight* W,
                                             const uint16_t* bias, const uint16_t* residual, int64_t ldr,
                                             uint32_t epilogue, float qscale, int64_t qscale_cols, void* C,
                                             int64_t ldc, void* stream) {
  clear_error();
  float* ws = nullptr;
  FQ_TRY(scratch_for_current_device(&ws));
  FixedWorkspaceScope scope(ws);
  return dequant_gemm(A, M, lda, W, bias, residual, ldr, epilogue, qscale, qscale_cols, C, ldc, stream, false);
}

extern "C" fq_status fq_qkv_gemm_append(const uint16_t* A, int64_t M, int64_t lda, const fq_weight* W,
                                        const uint16_t* bias, float qscale, const fq_kv_layer* kv, int64_t b0,
                                        int64_t B, int64_t T, int64_t pos, uint16_t* C, int64_t ldc, void* stream) {
  clear_error();
  FQ_CHECK_ARG(W != nullptr && kv != nullptr, "fq_qkv_gemm_append: NULL W or kv");
  FQ_CHECK_ARG(kv_bits_valid(*kv), "fq_qkv_gemm_append: bits must be 4 or 16");
  FQ_CHECK_ARG(kv->head_dim > 0 && kv->head_dim % 64 == 0 && kv->heads > 0,
               "fq_qkv_gemm_append: head_dim must be a positive multiple of 64");
  const int64_t h = (int64_t)kv->heads * kv->head_dim;
  FQ_CHECK_ARG(W->n == 3 * h, "fq_qkv_gemm_append: W must have 3 * heads * head_dim rows");
  FQ_CHECK_ARG(B >= 0 && T >= 0 && M == B * T, "fq_qkv_gemm_append: M must equal B * T");
  FQ_CHECK_ARG(b0 >= 0 && pos >= 0 && b0 + B <= kv->batch && pos + T <= kv->capacity,
               "fq_qkv_gemm_append: sequences or positions exceed the cache");
  const uint32_t flags = (bias ? FQ_EPI_BIAS : 0u) | FQ_EPI_QSCALE;
  const bool f16 = kv_is_f16(*kv);
  const bool cache_ok = f16 ? (kv->k16 && kv->v16 && (uintptr_t)kv->k16 % 16 == 0 && (uintptr_t)kv->v16 % 16 == 0)
                            : (kv->k_codes && kv->v_codes && kv->k_meta && kv->v_meta &&
                               (uintptr_t)kv->k_codes % 8 == 0 && (uintptr_t)kv->v_codes % 8 == 0 &&
                               (uintptr_t)kv->k_meta % 4 == 0 && (uintptr_t)kv->v_meta % 4 == 0);
  const bool fused = M > 0 && tile256_fits(M, W->n, W->k, lda, W) && cache_ok &&
                     (!bias || (uintptr_t)bias % 16 == 0) && kv->group == FQ_GROUP;
  if (!fused) {
    // unfused: the projection into C, then the append kernel reads K and V back
    FQ_TRY(fq_dequant_gemm(A, M, lda, W, bias, nullptr, 0, flags, qscale, h, C, ldc, stream));
    if (M == 0) return FQ_OK;
    return fq_kv_append(kv, C + h, C + 2 * h, ldc, b0, B, T, pos, stream);
  }
  const int64_t N = W->n, K = W->k;
  FQ_CHECK_ARG(K % 64 == 0 && lda >= K && lda % 8 == 0 && ldc >= N, "fq_qkv_gemm_append: bad K or strides");
  FQ_CHECK_ARG(W->packed.group == FQ_GROUP && W->packed.rows == N && W->packed.cols == K && W->packed.codes &&
                   W->packed.meta && (uintptr_t)W->packed.codes % 16 == 0 && (uintptr_t)W->packed.meta % 4 == 0,
               "fq_qkv_gemm_append: bad packed weight");
  FQ_CHECK_ARG(A && C && (uintptr_t)A % 16 == 0, "fq_qkv_gemm_append: NULL or misaligned A / C");
  Epilogue epi{bias, nullptr, 0, flags, qscale, h, C, ldc};
  KvAppend kva{kv->k_codes, kv->k_meta, kv->v_codes, kv->v_meta, kv->k16, kv->v16, h, kv->capacity, b0, pos,
               (int)T, kv->heads, kv->head_dim, f16 ? 1 : 0};
  hipStream_t st = as_stream(stream);
  const int tk = timing_begin(FQ_KC_GEMM_PREFILL, st);
  const dim3 grid((unsigned)(ceil_div(M, 256) * ceil_div(N, 256)));
  gemm_w4_kernel<true><<<grid, dim3(256), 0, st>>>(A, M, lda, W->packed.codes, W->packed.meta, N, K, epi, kva);
  FQ_TRY(launch_check("gemm_w4_kernel"));
  if (tk >= 0) {
    const double bytes = 2.0 * M * K + 0.5625 * N * K + 2.0 * M * h + (f16 ? 2.0 : 0.5625) * 2.0 * M * h + 2.0 * N;
    timing_end(tk, FQ_KC_GEMM_PREFILL, 2.0 * M * N * K, bytes, st);
  }
  return FQ_OK;
}
