// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built with the library's sources compiled for
// the host only, run on a machine without a GPU).  Every entry point is
// called with invalid arguments (each must be rejected with its status and
// launch nothing) and with valid ones (they pass validation and stop at the
// device check, HBL_ERR_DEVICE, since no GPU is present); the workspace
// sizing is evaluated over the whole shape range.  The sanitizers flag any
// out-of-bounds access, signed overflow or other undefined behaviour in that
// host code.  Prints "ok" and exits 0 when every expectation holds.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hbl.h"
#include "hbl_attn.h"

static int fails = 0;
#define EXPECT(call, want)                                                                         \
  do {                                                                                             \
    const int got_ = (int)(call);                                                                  \
    if (got_ != (int)(want)) {                                                                     \
      std::printf("FAIL line %d: %s -> %d, want %d\n", __LINE__, #call, got_, (int)(want));          \
      ++fails;                                                                                     \
    }                                                                                              \
  } while (0)

alignas(256) static unsigned char buf[1 << 16];

int main() {
  void* A = buf;
  void* B = buf + 4096;
  void* BAD = buf + 1;
  float* F = reinterpret_cast<float*>(buf + 8192);
  uint8_t* U = buf + 12288;
  const hipStream_t S = nullptr;
  const size_t BIG = (size_t)1 << 40;

  // status strings: every code has a distinct message
  for (int s = 0; s <= 8; ++s) {
    const char* m = hbl_status_string((hbl_status)s);
    if (!m || !*m) { std::printf("FAIL status string %d\n", s); ++fails; }
  }

  // workspace sizing over the whole shape range (no overflow, monotone in M)
  const int ops[] = {HBL_OP_QUANTIZE_WEIGHTS, HBL_OP_MATMUL, HBL_OP_QUANTIZE_WEIGHTS_ROTATED, HBL_OP_FORWARD_INT4,
                     HBL_OP_FORWARD_INT8, HBL_OP_BACKWARD, 3, 99, -1};
  const int64_t Ms[] = {0, 1, 3, 4, 5, 16, 17, 32, 33, 64, 65, 255, 256, 257, 8192, 65537, (int64_t(1) << 24)};
  const int64_t Ns[] = {16, 48, 272, 4096, 11008, (int64_t(1) << 20)};
  for (int op : ops)
    for (int64_t K = 64; K <= 32768; K *= 2)
      for (int64_t N : Ns) {
        size_t prev = 0;
        for (int64_t M : Ms) {
          if (M * (K > N ? K : N) >= (int64_t(1) << 40)) continue;
          const size_t w = hbl_workspace_bytes(op, M, K, N);
          if ((op == HBL_OP_FORWARD_INT8 || op == HBL_OP_FORWARD_INT4) && M > 65 && w < prev) {
            std::printf("FAIL workspace not monotone op %d M %lld K %lld N %lld\n", op, (long long)M, (long long)K,
                        (long long)N);
            ++fails;
          }
          if (w % 256 && w) { std::printf("FAIL workspace not 256-aligned\n"); ++fails; }
          prev = w;
        }
      }
  EXPECT(hbl_workspace_bytes(HBL_OP_MATMUL, -1, 256, 256), 0);
  EXPECT(hbl_workspace_bytes(HBL_OP_MATMUL, 1, 0, 256), 0);
  EXPECT(hbl_attention_workspace_bytes(0, 8, 128, 100), 0);
  EXPECT(hbl_attention_workspace_bytes(2, 8, 96, 100), 0);
  (void)hbl_attention_workspace_bytes(64, 64, 256, int64_t(1) << 24);

  // forward: every rejection, then valid arguments (stop at the device check)
  for (int bits : {8, 4}) {
    auto fwd = [&](const void* x, int xd, const float* g, const void* wp, const void* wa, int64_t M, int64_t K,
                   int64_t N, void* y, int yd, void* ws, size_t wsb) {
      return bits == 8 ? hbl_forward_int8(x, (hbl_dtype)xd, g, (const uint8_t*)wp, (const float*)wa, M, K, N, y,
                                          (hbl_dtype)yd, ws, wsb, S)
                       : hbl_forward_int4(x, (hbl_dtype)xd, g, (const uint8_t*)wp, (const float*)wa, M, K, N, y,
                                          (hbl_dtype)yd, ws, wsb, S);
    };
    EXPECT(fwd(nullptr, 1, nullptr, A, A, 8, 256, 256, B, 1, A, BIG), HBL_ERR_NULL);
    EXPECT(fwd(A, 1, nullptr, nullptr, A, 8, 256, 256, B, 1, A, BIG), HBL_ERR_NULL);
    EXPECT(fwd(A, 1, nullptr, A, A, 8, 256, 256, nullptr, 1, A, BIG), HBL_ERR_NULL);
    EXPECT(fwd(A, 1, nullptr, A, A, 8, 256, 256, B, 1, nullptr, BIG), HBL_ERR_NULL);
    EXPECT(fwd(A, 7, nullptr, A, A, 8, 256, 256, B, 1, A, BIG), HBL_ERR_DTYPE);
    EXPECT(fwd(A, 1, nullptr, A, A, 8, 256, 256, B, -3, A, BIG), HBL_ERR_DTYPE);
    for (int64_t K : {0, 32, 48, 300, 65536, -256}) EXPECT(fwd(A, 1, nullptr, A, A, 8, K, 256, B, 1, A, BIG), HBL_ERR_SHAPE);
    for (int64_t N : {0, 8, 250, -16}) EXPECT(fwd(A, 1, nullptr, A, A, 8, 256, N, B, 1, A, BIG), HBL_ERR_SHAPE);
    EXPECT(fwd(A, 1, nullptr, A, A, -1, 256, 256, B, 1, A, BIG), HBL_ERR_SHAPE);
    EXPECT(fwd(A, 1, nullptr, A, A, int64_t(1) << 31, 256, 256, B, 1, A, BIG), HBL_ERR_SHAPE);
    EXPECT(fwd(A, 1, nullptr, A, A, int64_t(1) << 28, 16384, 256, B, 1, A, BIG), HBL_ERR_SHAPE);
    EXPECT(fwd(BAD, 1, nullptr, A, A, 8, 256, 256, B, 1, A, BIG), HBL_ERR_ALIGN);
    EXPECT(fwd(A, 1, (const float*)BAD, A, A, 8, 256, 256, B, 1, A, BIG), HBL_ERR_ALIGN);
    EXPECT(fwd(A, 1, nullptr, A, A, 8, 256, 256, B, 1, BAD, BIG), HBL_ERR_ALIGN);
    EXPECT(fwd(A, 1, nullptr, A, A, 8, 256, 256, B, 1, A, 16), HBL_ERR_WORKSPACE);
    EXPECT(fwd(nullptr, 1, nullptr, nullptr, nullptr, 0, 256, 256, nullptr, 1, nullptr, 0), HBL_OK);
    for (int64_t K = 64; K <= 32768; K *= 2)
      for (int64_t M : {1, 4, 5, 16, 33, 64, 65, 300})
        EXPECT(fwd(A, 1, F, A, A, M, K, 272, B, 0, A, BIG), HBL_ERR_DEVICE);
    EXPECT(hbl_bitlinear_forward(A, HBL_BF16, nullptr, U, F, 8, 256, 256, bits, B, HBL_BF16, A, BIG, S),
           HBL_ERR_DEVICE);
    EXPECT(hbl_forward_noalloc(bits, A, HBL_BF16, nullptr, U, F, 8, 256, 256, B, HBL_BF16, S), HBL_ERR_DEVICE);
    EXPECT(hbl_forward_noalloc(bits, A, HBL_BF16, nullptr, U, F, 8192, 16384, 4096, B, HBL_BF16, S),
           HBL_ERR_SCRATCH);
  }
  EXPECT(hbl_bitlinear_forward(A, HBL_BF16, nullptr, U, F, 8, 256, 256, 5, B, HBL_BF16, A, BIG, S), HBL_ERR_DTYPE);
  EXPECT(hbl_forward_noalloc(6, A, HBL_BF16, nullptr, U, F, 8, 256, 256, B, HBL_BF16, S), HBL_ERR_DTYPE);

  // weights
  EXPECT(hbl_quantize_weights(F, 256, 255, U, F, A, BIG, S), HBL_ERR_SHAPE);
  EXPECT(hbl_quantize_weights(F, 256, 256, U, F, A, 8, S), HBL_ERR_WORKSPACE);
  EXPECT(hbl_quantize_weights(nullptr, 256, 256, U, F, A, BIG, S), HBL_ERR_NULL);
  EXPECT(hbl_quantize_weights(F, 256, 256, U, F, A, BIG, S), HBL_ERR_DEVICE);
  EXPECT(hbl_quantize_weights_rotated(F, 64, 1000, U, F, A, BIG, S), HBL_ERR_SHAPE);
  EXPECT(hbl_quantize_weights_rotated((const float*)BAD, 64, 1024, U, F, A, BIG, S), HBL_ERR_ALIGN);
  EXPECT(hbl_quantize_weights_rotated(F, 64, 32768, U, F, A, BIG, S), HBL_ERR_DEVICE);
  EXPECT(hbl_unpack_weights(U, 16, 256, nullptr, S), HBL_ERR_NULL);
  EXPECT(hbl_unpack_weights(U, 16, 64, (int8_t*)A, S), HBL_ERR_DEVICE);

  // stages
  for (int bits : {8, 4, 6}) {
    EXPECT(hbl_quantize_act(A, HBL_BF16, nullptr, 4, 200, bits, A, F, S), HBL_ERR_SHAPE);
    EXPECT(hbl_quantize_act(A, HBL_BF16, nullptr, 4, 256, bits, BAD, F, S), HBL_ERR_ALIGN);
    EXPECT(hbl_quantize_act(A, HBL_BF16, nullptr, 0, 256, bits, nullptr, nullptr, S), HBL_OK);
    EXPECT(hbl_quantize_act(A, HBL_BF16, nullptr, 4, 128, bits, A, F, S), bits == 6 ? HBL_ERR_SHAPE : HBL_ERR_DEVICE);
    EXPECT(hbl_quantize_act_unrotated(A, HBL_F32, F, 3, 32768, bits, A, F, S), HBL_ERR_DEVICE);
    EXPECT(hbl_quantize_rotated(F, 4, 200, bits, A, F, S), HBL_ERR_SHAPE);
    EXPECT(hbl_quantize_rotated(F, 0, 256, bits, nullptr, nullptr, S), HBL_OK);
    EXPECT(hbl_quantize_rotated(F, 4, 128, bits, A, F, S), bits == 6 ? HBL_ERR_SHAPE : HBL_ERR_DEVICE);
    EXPECT(hbl_quantize_rotated(F, 4, 256, bits, A, nullptr, S), HBL_ERR_NULL);
    EXPECT(hbl_gemm_ternary(A, bits, U, 4, 256, 250, (int32_t*)A, nullptr, 0, S), HBL_ERR_SHAPE);
    EXPECT(hbl_gemm_ternary(A, bits, U, 300, 64, 256, (int32_t*)A, nullptr, 0, S),
           bits == 6 ? HBL_ERR_SHAPE : HBL_ERR_DEVICE);
    EXPECT(hbl_gemm_ternary(A, bits, U, 64, 1024, 256, (int32_t*)A, nullptr, 0, S), HBL_ERR_NULL);
    EXPECT(hbl_matmul_dequant(A, bits, nullptr, U, F, 100, 256, 256, B, HBL_BF16, nullptr, 0, S), HBL_ERR_NULL);
    EXPECT(hbl_matmul_dequant(A, bits, F, U, F, 100, 32768, 256, B, HBL_F32, nullptr, 0, S), HBL_ERR_DEVICE);
  }
  EXPECT(hbl_quantize_act(A, HBL_BF16, nullptr, 4, 256, 5, A, F, S), HBL_ERR_DTYPE);
  EXPECT(hbl_rmsnorm_fwht(A, HBL_BF16, nullptr, 4, 256, (float*)BAD, S), HBL_ERR_ALIGN);
  EXPECT(hbl_rmsnorm_fwht(A, HBL_BF16, nullptr, 4, 64, F, S), HBL_ERR_DEVICE);

  // backward
  EXPECT(hbl_backward_weights(U, 16, 256, A, S), HBL_ERR_SHAPE);   // N % 32
  EXPECT(hbl_backward_weights(U, 32, 64, A, S), HBL_ERR_DEVICE);
  EXPECT(hbl_backward(A, HBL_BF16, nullptr, A, 8, F, A, F, A, 8, 256, 48, 1, A, HBL_F32, F, nullptr, A, BIG, S),
         HBL_ERR_SHAPE);
  EXPECT(hbl_backward(A, HBL_BF16, nullptr, A, 5, F, A, F, A, 8, 256, 64, 1, A, HBL_F32, F, nullptr, A, BIG, S),
         HBL_ERR_DTYPE);
  EXPECT(hbl_backward(A, HBL_BF16, nullptr, A, 4, F, A, F, A, 8, 256, 64, 1, A, HBL_F32, F, F, A, BIG, S),
         HBL_ERR_NULL);   // dgain without gain
  EXPECT(hbl_backward(A, HBL_BF16, F, A, 4, F, A, F, A, 8, 256, 64, 1, A, HBL_F32, F, F, A, 16, S),
         HBL_ERR_WORKSPACE);
  for (int64_t K = 64; K <= 32768; K *= 2)
    EXPECT(hbl_backward(A, HBL_BF16, F, A, 4, F, A, F, A, 70, K, 64, 1, A, HBL_F32, F, F, A, BIG, S),
           HBL_ERR_DEVICE);

  // low-bit attention states
  EXPECT(hbl_quantize_heads(nullptr, 4, 128, 5, nullptr, nullptr, S), HBL_ERR_DTYPE);
  EXPECT(hbl_quantize_heads(A, 4, 96, 3, U, F, S), HBL_ERR_SHAPE);
  EXPECT(hbl_quantize_heads(A, 4, 128, 3, U, F, S), HBL_ERR_DEVICE);
  EXPECT(hbl_dequantize_heads(U, F, 4, 128, 3, B, HBL_BF16, S), HBL_ERR_DEVICE);
  EXPECT(hbl_kv_cache_append(A, B, 1, 1, 2, 128, 3, nullptr, 0, U, F, U, F, S), HBL_ERR_SHAPE);
  EXPECT(hbl_kv_cache_append(A, B, 1, 1, 2, 128, 3, nullptr, 16, U, F, U, F, S), HBL_ERR_DEVICE);
  EXPECT(hbl_attention_decode(A, 8, U, F, U, F, 3, (const int32_t*)A, 1, 3, 2, 128, 16, B, HBL_BF16, nullptr, 0, S),
         HBL_ERR_SHAPE);
  EXPECT(hbl_attention_decode(A, 8, U, F, U, F, 3, (const int32_t*)A, 2, 8, 2, 128, 100000, B, HBL_BF16, A, BIG, S),
         HBL_ERR_DEVICE);
  EXPECT(hbl_attention_prefill(A, 8, U, F, U, F, 3, (const int32_t*)A, 1, (int64_t(1) << 31) - 600, 4, 2, 128, 100,
                               B, HBL_BF16, S),
         HBL_ERR_SHAPE);
  EXPECT(hbl_attention_prefill(A, 8, U, F, U, F, 3, (const int32_t*)A, 2, 64, 4, 2, 128, 4096, B, HBL_BF16, S),
         HBL_ERR_DEVICE);

  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
