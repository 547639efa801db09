// Host-side launch descriptors shared by the C ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hbl.h"

namespace hbl {

// Every check of the forward's arguments except the workspace's (host only,
// touches no device): HBL_OK or the first error.
hbl_status forward_check(int bits, const void* x, hbl_dtype x_dtype, const float* gain, const uint8_t* w_packed,
                         const float* w_alpha, int64_t M, int64_t K, int64_t N, const void* y, hbl_dtype y_dtype);

struct PrepArgs {
  const void* x;
  bool x_bf16;
  const float* gain;
  int M;
  int cus;           // compute units of the device (persistent grid size)
  int logk;
  int bits;          // 8 or 4
  int mode;          // 0: codes + scales, 1: rotated activations (fp32),
                     // 2: INT4 codes in the fp6 operand layout + scales,
                     // 3: rows rotated without normalisation (fp32, x fp32)
  bool rotate;       // modes 0 and 2: false leaves the transform out
  bool blocked;      // mode 0: codes in the decode-blocked layout (dblk_offset), 5..64 tokens
  bool as_given;     // modes 0 and 2, fp32 x, no transform: quantise x as given
                     // (no RMSNorm either: x is already the rotated activation)
  uint8_t* codes;
  float* dscale;
  float* xt;
  uint32_t* zero;    // words the first workgroup clears (the matmul's split-K counters), or nullptr
  int nzero;
  hipStream_t stream;
};
hipError_t launch_prep(const PrepArgs& a);

enum OutKind { OUT_ACC_I32 = 0, OUT_F32 = 1, OUT_BF16 = 2 };

struct GemmArgs {
  const uint8_t* codes;   // int8 [M][K] or int4 [M][K/2]
  int bits;
  const uint8_t* wpack;   // [N][K/4]
  const float* dscale;    // [M]   (unused for OUT_ACC_I32)
  const float* walpha;    // [1]   (unused for OUT_ACC_I32)
  void* out;
  int out_kind;
  int M, N, K;
  void* ws;               // split-K partials (decode path)
  size_t ws_bytes;
  uint32_t* tile_count;   // zeroed split-K arrival counters (or nullptr: separate reduction kernel)
  bool codes_blocked;     // codes in the decode-blocked layout (5..64 tokens, K >= 512, bits 8 or 4)
  hipStream_t stream;
};
hipError_t launch_gemm(const GemmArgs& a);
// INT4 on the fp6 x fp4 matrix instruction: codes in the fp6 operand layout
// that prep mode 2 writes, [K/128][M][96].  Up to 64 tokens the split decode
// matmul runs it, beyond that the prefill matmul; the INT4 forward takes this
// path for M > kFp6MinM only (at 64 tokens and fewer the int8 decode matmul
// measured faster).
constexpr int kFp6MinM = 64;
// The fp6 operand layout is blocked by 128 k and its matmul stages two such
// blocks per step, so format 6 needs K >= 256 (shorter rows use format 4).
constexpr int kFp6MinK = 256;
hipError_t launch_gemm_fp6(const GemmArgs& a);
// Workspace bytes the matmul needs beyond the codes and scales (blocked: the
// codes come in the decode-blocked layout, which changes the plan for 33-64
// tokens).
size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N, bool blocked);
// Split-K arrival counters inside that workspace (count 0 / nullptr when the
// shape needs none); they must be zero when the matmul starts.
int gemm_tile_counters(int64_t M, int64_t K, int64_t N, bool blocked);
uint32_t* gemm_tile_counter_ptr(void* ws, int64_t M, int64_t K, int64_t N, bool blocked);

// Single-launch forward for 1..4 tokens with K = 8192 or 16384 (decode):
// transform, quantiser and matmul in one kernel.
struct FusedDecodeArgs {
  const void* x;
  bool x_bf16;
  const float* gain;
  const uint8_t* wpack;
  const float* walpha;
  void* out;
  int out_kind;           // OUT_F32 or OUT_BF16
  int M, N, logk, bits;
  bool rotate;            // false: BitLinear without the transform
  hipStream_t stream;
};
bool decode_fused_supported(int M, int logk, bool rotate);
hipError_t launch_decode_fused(const FusedDecodeArgs& a);

struct WquantArgs {
  const float* w;
  int N, K;
  uint8_t* wpack;
  float* walpha;
  double* rowsum;         // workspace [N]
  hipStream_t stream;
};
hipError_t launch_wquant(const WquantArgs& a);
hipError_t launch_unpack(const uint8_t* wpack, int N, int K, int8_t* wt, hipStream_t stream);

// Low-bit attention states: per-head absmax codes of post-RoPE Q/K/V.
struct QuantHeadsArgs {
  const void* x0;         // bf16 [B][Tn][H][d]
  const void* x1;         // optional second tensor of the same shape (V beside K)
  uint8_t* codes0;        // packed rows [B][H][Tmax][d*bits/8]
  uint8_t* codes1;
  float* scale0;          // [B][H][Tmax]
  float* scale1;
  int64_t B, H, Tn, Tmax;
  const int32_t* pos;     // device [B] first cache position per sequence, or NULL (0)
  int d, bits;
  hipStream_t stream;
};
hipError_t launch_quant_heads(const QuantHeadsArgs& a);
hipError_t launch_dequant_heads(const uint8_t* codes, const float* scale, int64_t R, int d, int bits, void* y,
                                bool y_bf16, hipStream_t stream);

struct AttnArgs {
  const void* q;          // bf16 [B][Hq][d]
  int qbits;
  const uint8_t* kc;      // packed [B][Hkv][Tmax][d*kvbits/8]
  const float* ks;        // [B][Hkv][Tmax]
  const uint8_t* vc;
  const float* vs;
  int kvbits;
  const int32_t* lens;    // device [B]
  int B, Hq, Hkv, d;
  int64_t Tmax;
  int ct, nchunk;         // tokens per chunk and chunks per head (attn_plan)
  float* part;            // [B][Hq][nchunk][attn_part_stride(d)]
  void* out;              // [B][Hq][d]
  bool out_bf16;
  hipStream_t stream;
};
bool heads_bits_supported(int bits);
// Chunking of the cached tokens: one chunk per head when the heads give at
// least 512 workgroups (two per compute unit of a 256-CU part), otherwise
// enough chunks to reach that, in whole blocks of attn_block_tokens(d).
int attn_block_tokens(int d);
void attn_plan(int64_t B, int64_t Hq, int d, int64_t Tmax, int* ct, int* nchunk);
hipError_t launch_attention_decode(const AttnArgs& a);
struct PrefillArgs {
  const void* q;          // bf16 [B][Tn][Hq][d]
  int qbits;
  const uint8_t* kc;      // packed [B][Hkv][Tmax][d*kvbits/8]
  const float* ks;
  const uint8_t* vc;
  const float* vs;
  int kvbits;
  const int32_t* start;   // device [B]: position of each sequence's first new token
  int B, Tn, Hq, Hkv, d;
  int64_t Tmax;
  void* out;              // [B][Tn][Hq][d]
  bool out_bf16;
  hipStream_t stream;
};
hipError_t launch_attention_prefill(const PrefillArgs& a);

// Backward pass (straight-through estimator).
struct BwdArgs {
  const float* dxh;       // [M][K] fp32: gradient at the quantiser input
  const void* x;          // [M][K] the forward's input
  bool x_bf16;
  const float* gain;      // [K] or NULL
  int M, logk;
  void* dx;               // [M][K]
  bool dx_bf16;
  bool rotate;
  hipStream_t stream;
};
int bwd_prep_tpb(int logk);
hipError_t launch_wbt(const uint8_t* wpack, int N, int K, uint16_t* wbt, hipStream_t stream);
hipError_t launch_transpose_tokens(int kind, const void* src, const float* dscale, int M, int C, int Mp,
                                   uint16_t* dst, hipStream_t stream);
hipError_t launch_gemm_bf16_nt(const uint16_t* A, const uint16_t* B, const float* scale, float* out, int I, int J,
                               int Cn, hipStream_t stream);
hipError_t launch_bwd_prep(const BwdArgs& a, int grid, float* dgpart);
hipError_t launch_dg_reduce(const float* part, int rows, int K, float* dg, hipStream_t stream);
int attn_part_stride(int d);

}  // namespace hbl
