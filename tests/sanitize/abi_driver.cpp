// Drives the host side of every C-ABI entry point -- argument validation,
// size queries and empty-batch no-ops, none of which launches a kernel -- so
// that a host build with AddressSanitizer and UndefinedBehaviorSanitizer can
// check it.  Prints "ok" on success.
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "moe_fp8.h"

#define EXPECT(cond)                                                 \
    do {                                                             \
        if (!(cond)) {                                               \
            std::printf("failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                                \
        }                                                            \
    } while (0)

int main() {
    // a non-null, 256-byte aligned address that is never dereferenced on the host
    void* fake = reinterpret_cast<void*>(uintptr_t{0x10000});
    auto* f32 = static_cast<float*>(fake);
    auto* i64 = static_cast<int64_t*>(fake);
    auto* i32 = static_cast<int32_t*>(fake);
    auto* u16 = static_cast<uint16_t*>(fake);
    auto* u8 = static_cast<uint8_t*>(fake);
    const moe_status bad = MOE_ERR_INVALID_ARGUMENT;
    EXPECT(moe_topk_gate(nullptr, 4, 16, 2, 0, i64, nullptr, nullptr) == bad);
    EXPECT(moe_topk_gate(f32, 4, 16, 17, 0, i64, nullptr, nullptr) == bad);
    EXPECT(moe_topk_gate(nullptr, 0, 16, 2, 0, nullptr, nullptr, nullptr) == MOE_OK);
    EXPECT(moe_token_map_workspace_bytes(1000, 8, 256) > 0);
    EXPECT(moe_token_map_workspace_bytes(-1, 8, 256) == 0);
    EXPECT(moe_token_map(i64, 1000, 8, 256, i32, i32, i32, nullptr, fake, 1, nullptr) ==
           MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_token_map(i64, 1000, 0, 256, i32, i32, i32, nullptr, fake, 1 << 20, nullptr) == bad);
    EXPECT(moe_expand_cast_fp8(u16, 64, 1000, 4, i32, nullptr, 256, 128, u8, f32, nullptr, nullptr) == bad);
    EXPECT(moe_expand_cast_fp8(u16, 64, 1024, 4, i32, nullptr, 256, 64, u8, f32, nullptr, nullptr) ==
           MOE_ERR_UNSUPPORTED);
    EXPECT(moe_expand_cast_fp8(nullptr, 0, 1024, 4, i32, nullptr, 0, 128, nullptr, nullptr, nullptr, nullptr) ==
           MOE_OK);
    EXPECT(swiglu_cast_fp8(u16, 64, 2048, nullptr, NAN, 128, u8, f32, nullptr) == bad);
    EXPECT(swiglu_cast_fp8(nullptr, 0, 2048, nullptr, 0.0f, 128, nullptr, nullptr, nullptr) == MOE_OK);
    EXPECT(moe_combine(u16, 16, 100, i32, nullptr, 8, 2, u16, nullptr) == bad);
    EXPECT(moe_combine(nullptr, 0, 256, nullptr, nullptr, 0, 2, nullptr, nullptr) == MOE_OK);
    EXPECT(moe_token_map_aligned_rows(1000, 8, 32, 128) == 1000 * 8 + 32 * 127);
    EXPECT(moe_token_map_aligned(i64, 1000, 8, 64, 32, 128, i32, i32, i32, i32, 1 << 20, fake, 1 << 20,
                                 nullptr) == bad);
    EXPECT(moe_expand_cast_fp8_padded(u16, 64, 1024, 4, nullptr, nullptr, i32, 512, 128, u8, f32, nullptr,
                                      nullptr) == bad);
    moe_cast_format fmt{MOE_FMT_E2M1, 32, 1, 1, 0.0f};
    EXPECT(moe_expand_cast(u16, 64, 1040, 4, i32, nullptr, 256, &fmt, u8, fake, nullptr, nullptr) == bad);
    fmt.clamp_min = 1e-38f;
    EXPECT(moe_expand_cast(u16, 64, 1024, 4, i32, nullptr, 256, &fmt, u8, fake, nullptr, nullptr) == bad);
    EXPECT(swiglu_cast(u16, 64, 2048, nullptr, 0.0f, nullptr, u8, fake, nullptr) == bad);
    EXPECT(moe_dispatch_workspace_bytes(64, 8, 256) >= 2048);
    EXPECT(moe_dispatch(f32, u16, 64, 256, 8, 7168, 0, 128, i64, nullptr, i32, i32, i32, nullptr, u8, f32,
                        nullptr, fake, 1 << 20, 7, nullptr) == bad);
    EXPECT(moe_route_workspace_bytes(4096, 8, 256) == moe_dispatch_workspace_bytes(4096, 8, 256));
    EXPECT(moe_route_workspace_bytes(4096, 0, 256) == 0);
    EXPECT(moe_route(f32, 4096, 256, 8, 0, i64, nullptr, i32, i32, i32, nullptr, fake, 1 << 24, 4, nullptr) == bad);
    EXPECT(moe_route(f32, 33, 256, 8, 0, i64, nullptr, i32, i32, i32, nullptr, fake, 1 << 24, MOE_ROUTE_LOCAL,
                     nullptr) == MOE_ERR_UNSUPPORTED);
    EXPECT(moe_route(f32, 4096, 256, 8, 1, i64, nullptr, i32, i32, i32, nullptr, fake, 1 << 24, 0, nullptr) == bad);
    EXPECT(moe_route(f32, 4096, 256, 8, 0, i64, nullptr, i32, i32, i32, nullptr, fake, 16, 0, nullptr) ==
           MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_route(f32, 1 << 20, 256, 8, 0, i64, nullptr, i32, i32, i32, nullptr, fake, size_t{1} << 32,
                     MOE_ROUTE_FUSED, nullptr) == MOE_ERR_UNSUPPORTED);
    EXPECT(moe_status_string(static_cast<moe_status>(99)) != nullptr);
    EXPECT(moe_fp8_version() >= 200);
    std::puts("ok");
    return 0;
}
