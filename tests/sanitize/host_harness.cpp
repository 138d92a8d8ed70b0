// Host-side harness of the C ABI for the sanitizer build (ASan + UBSan, no
// GPU): every call is driven through its argument validation and its host
// arithmetic (workspace sizing, plan sizes, status text), with arguments
// chosen so that validation refuses them before any HIP call.  Exits 0 when
// every call returned the documented status.
#include <cstdio>
#include <cstring>

#include "moe_skinny.h"

static int g_bad = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
      ++g_bad;                                                        \
    }                                                                 \
  } while (0)

int main() {
  void* A = reinterpret_cast<void*>(0x10000);   // aligned, never dereferenced
  void* M = reinterpret_cast<void*>(0x10004);   // misaligned
  const size_t BIG = (size_t)1 << 34;
  EXPECT(moe_abi_version() == MOE_ABI_VERSION);
  for (int s = -1; s <= 6; ++s) EXPECT(std::strlen(moe_status_str(s)) > 0);
  // plan and workspace sizes over the whole scope and beyond
  for (int B = 0; B <= 70; B += 7)
    for (int k = 1; k <= 17; k += 4)
      for (int E = 1; E <= 520; E += 37) {
        if (B > 0) EXPECT(moe_plan_words(B, k, E) == 2 + 2 * (B * k < E ? B * k : E) + B * k);
        for (int op = -1; op <= 4; ++op)
          for (int dt = 0; dt <= 1; ++dt) {
            const size_t n = moe_workspace_bytes(op, dt, B, 16384, E, k, 256, 256, 3072, 7168);
            if (op == MOE_OP_BLOCK && B >= 1 && B <= 64 && E <= 512 && k <= 16 && dt == MOE_DT_BF16)
              EXPECT(n > 0 && n <= MOE_NOALLOC_SCRATCH_BYTES);
          }
      }
  EXPECT(moe_workspace_bytes(MOE_OP_SKINNY_GEMM, MOE_DT_BF16, 64, 0, 0, 0, 0, 0, 3072, -5) == 0);
  EXPECT(moe_workspace_status_offset() > 0);
  // variant / schedule switches round-trip and ignore unknown values
  const int pv = moe_set_variant(MOE_VARIANT_MFMA);
  EXPECT(moe_set_variant(99) == MOE_VARIANT_MFMA);
  EXPECT(moe_set_variant(pv) == MOE_VARIANT_MFMA);
  const int ps = moe_set_block_schedule(MOE_SCHEDULE_FUSED);
  EXPECT(moe_set_block_schedule(-3) == MOE_SCHEDULE_FUSED);
  moe_set_block_schedule(ps);
  EXPECT(moe_profile_events(42, A, A) == MOE_EINVAL);
  EXPECT(moe_profile_events(MOE_KERNEL_ROUTE, A, nullptr) == MOE_EINVAL);
  EXPECT(moe_profile_events(MOE_KERNEL_ROUTE, nullptr, nullptr) == MOE_OK);
  // skinny products
  EXPECT(skinny_gemm(7, 4, 64, 256, A, A, A, 1, A, BIG, nullptr) == MOE_EINVAL);
  EXPECT(skinny_gemm(MOE_DT_BF16, 0, 64, 256, A, A, A, 1, A, BIG, nullptr) == MOE_EINVAL);
  EXPECT(skinny_gemm(MOE_DT_BF16, 65, 64, 256, A, A, A, 1, A, BIG, nullptr) == MOE_EUNSUPPORTED);
  EXPECT(skinny_gemm(MOE_DT_BF16, 4, 64, 252, A, A, A, 1, A, BIG, nullptr) == MOE_EUNSUPPORTED);
  EXPECT(skinny_gemm(MOE_DT_BF16, 4, 64, 256, M, A, A, 1, A, BIG, nullptr) == MOE_EINVAL);
  EXPECT(skinny_gemm(MOE_DT_BF16, 64, 3072, 7168, A, A, A, 1, A, 16, nullptr) == MOE_EWORKSPACE);
  EXPECT(skinny_gemm_residual(MOE_DT_BF16, 4, 64, 256, A, A, nullptr, A, 1, A, BIG, nullptr) == MOE_EINVAL);
  EXPECT(std::strlen(moe_last_error()) > 0);
  // router
  EXPECT(moe_route(MOE_DT_BF16, 8, 7168, 384, 0, A, A, nullptr, 0, (int32_t*)A, (float*)A, (int32_t*)A, nullptr, A,
                   BIG, nullptr) == MOE_EINVAL);
  EXPECT(moe_route(MOE_DT_BF16, 8, 7168, 8, 9, A, A, nullptr, 0, (int32_t*)A, (float*)A, (int32_t*)A, nullptr, A,
                   BIG, nullptr) == MOE_EINVAL);
  EXPECT(moe_route(MOE_DT_BF16, 8, 7168, 513, 8, A, A, nullptr, 0, (int32_t*)A, (float*)A, (int32_t*)A, nullptr, A,
                   BIG, nullptr) == MOE_EUNSUPPORTED);
  EXPECT(moe_route(MOE_DT_BF16, 8, 7168, 384, 8, A, A, (const float*)A, 7, (int32_t*)A, (float*)A, (int32_t*)A,
                   nullptr, A, BIG, nullptr) == MOE_EINVAL);
  EXPECT(moe_route(MOE_DT_BF16, 64, 7168, 384, 8, A, A, nullptr, 0, (int32_t*)A, (float*)A, (int32_t*)A, nullptr, A,
                   1024, nullptr) == MOE_EWORKSPACE);
  // experts, combine, block
  EXPECT(moe_expert_ffn(MOE_DT_BF16, 8, 7168, 384, 8, 100, A, (const int32_t*)A, A, A, 128, A, A, (float*)A, A, BIG,
                        nullptr) == MOE_EUNSUPPORTED);
  EXPECT(moe_expert_ffn(MOE_DT_BF16, 8, 7168, 384, 8, 128, A, (const int32_t*)A, A, A, 128, A, nullptr, (float*)A, A,
                        BIG, nullptr) == MOE_EINVAL);
  EXPECT(moe_expert_ffn(MOE_DT_BF16, 8, 7168, 384, 8, 128, A, (const int32_t*)A, A, A, 128, A, A, (float*)A, A, 64,
                        nullptr) == MOE_EWORKSPACE);
  EXPECT(moe_combine(MOE_DT_BF16, 65, 7168, 8, (const float*)A, (const float*)A, 1, A, nullptr) == MOE_EUNSUPPORTED);
  EXPECT(moe_combine(MOE_DT_BF16, 1, 7168, 8, (const float*)A, (const float*)M, 1, A, nullptr) == MOE_EINVAL);
  EXPECT(moe_block(MOE_DT_BF16, 65, 7168, 384, 8, 128, 128, A, A, nullptr, 0, A, A, A, A, A, nullptr, nullptr, A, BIG,
                   nullptr) == MOE_EUNSUPPORTED);
  EXPECT(moe_block(MOE_DT_BF16, 1, 7168, 384, 8, 128, 128, A, A, nullptr, 0, A, A, A, A, M, nullptr, nullptr, A, BIG,
                   nullptr) == MOE_EINVAL);
  EXPECT(moe_block(MOE_DT_BF16, 1, 7168, 384, 8, 128, 128, A, A, nullptr, 0, A, A, A, A, A, nullptr, nullptr, A, 1000,
                   nullptr) == MOE_EWORKSPACE);
  EXPECT(moe_block_noalloc(MOE_DT_BF16, 1, 7168, 384, 8, 300, 128, A, A, nullptr, 0, A, A, A, A, A, nullptr, nullptr,
                           nullptr) == MOE_EUNSUPPORTED);
  EXPECT(moe_block_noalloc(MOE_DT_F32, 9, 1024, 16, 2, 64, 0, A, A, nullptr, 0, A, A, nullptr, nullptr, A, nullptr,
                           nullptr, nullptr) == MOE_EUNSUPPORTED);
  EXPECT(moe_stream_read(A, 0, (uint32_t*)A, 16, nullptr) == MOE_EINVAL);
  EXPECT(moe_stream_read(A, 4096, (uint32_t*)A, 0, nullptr) == MOE_EINVAL);
  EXPECT(moe_workspace_init(M, 4096, nullptr) == MOE_EINVAL);
  std::printf("host harness: %d failures\n", g_bad);
  return g_bad ? 1 : 0;
}
