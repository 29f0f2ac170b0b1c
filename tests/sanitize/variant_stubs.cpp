// Stand-ins for the kernel variant tables, so that the host-side plan code (api.cpp) links into the
// sanitizer build without any device code: every request reports "no kernel variant".
#include <cstdint>

namespace bsg {
struct KernelVariant;
const KernelVariant* mxfp8_variants(int64_t, int64_t, int64_t, int64_t, bool) { return nullptr; }
const KernelVariant* nvfp4_variants(int64_t, int64_t, int64_t, int64_t) { return nullptr; }
}  // namespace bsg
