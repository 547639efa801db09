// Host-side launch descriptors shared by the C ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hbl {

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
  uint8_t* codes;
  float* dscale;
  float* xt;
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
  hipStream_t stream;
};
hipError_t launch_gemm(const GemmArgs& a);
// INT4 prefill on the fp6 x fp4 matrix instruction: codes in the fp6 operand
// layout that prep mode 2 writes, [M][K*3/4].  Used for M > kFp6MinM.
constexpr int kFp6MinM = 64;
hipError_t launch_gemm_fp6(const GemmArgs& a);
// Workspace bytes the matmul needs beyond the codes and scales.
size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N);

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
bool decode_fused_supported(int M, int logk);
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

}  // namespace hbl
