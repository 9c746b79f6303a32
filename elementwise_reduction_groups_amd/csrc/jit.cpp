// hipRTC compilation of emitted kernels for gfx950.
//
// Flags: -O3; -ffp-contract=off so no multiply-add is fused (the oracle and
// the pages' kernels round every operation, and fusion keeps the operation
// order: PSK-Realize, "What it buys, measured"); correctly rounded f32
// division and square root; packed-FP32
// instructions disabled.  hipRTC needs no GPU, so kernels also compile in a
// host-only process.
#include <hip/hiprtc.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "psk_internal.h"

namespace psk {

const char* const kJitOptions[] = {
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
};
const int kJitOptionCount = (int)(sizeof(kJitOptions) / sizeof(kJitOptions[0]));

static std::string cache_path(const std::string& source)
{
    const char* dir = std::getenv("PSK_CACHE_DIR");
    if (!dir || !*dir) return std::string();
    std::string key = source;
    for (int i = 0; i < kJitOptionCount; ++i) key += kJitOptions[i];
    char name[64];
    std::snprintf(name, sizeof name, "/psk_%016llx.co", (unsigned long long)fnv1a(key));
    return std::string(dir) + name;
}

// The code object's metadata is a MessagePack map in an ELF note; the kernel
// descriptor's ".private_segment_fixed_size" key is followed by an unsigned
// integer (positive fixint, or uint8/16/32/64 with their markers).
int64_t code_scratch_bytes(const std::vector<char>& code)
{
    static const char key[] = ".private_segment_fixed_size";
    const size_t kl = sizeof key - 1;
    for (size_t i = 0; i + kl + 9 < code.size(); ++i) {
        if (std::memcmp(code.data() + i, key, kl) != 0) continue;
        const unsigned char* p = reinterpret_cast<const unsigned char*>(code.data() + i + kl);
        const unsigned m = p[0];
        if (m <= 0x7f) return m;
        int n = m == 0xcc ? 1 : m == 0xcd ? 2 : m == 0xce ? 4 : m == 0xcf ? 8 : 0;
        if (!n) return -1;
        int64_t v = 0;
        for (int k = 1; k <= n; ++k) v = (v << 8) | p[k];   // MessagePack integers are big-endian
        return v;
    }
    return -1;
}

psk_status jit_compile(const std::string& source, const std::string& name, std::vector<char>& code)
{
    std::string cpath = cache_path(source);
    if (!cpath.empty()) {
        if (FILE* f = std::fopen(cpath.c_str(), "rb")) {
            std::fseek(f, 0, SEEK_END);
            long sz = std::ftell(f);
            std::fseek(f, 0, SEEK_SET);
            code.resize(sz > 0 ? (size_t)sz : 0);
            bool ok = sz > 0 && std::fread(code.data(), 1, (size_t)sz, f) == (size_t)sz;
            std::fclose(f);
            if (ok) {
                count_jit(true);
                return PSK_OK;
            }
        }
    }
    hiprtcProgram prog;
    std::string fname = name + ".hip";
    hiprtcResult r = hiprtcCreateProgram(&prog, source.c_str(), fname.c_str(), 0, nullptr, nullptr);
    if (r != HIPRTC_SUCCESS) return fail(PSK_E_JIT, std::string("hiprtcCreateProgram: ") + hiprtcGetErrorString(r));
    r = hiprtcCompileProgram(prog, kJitOptionCount, kJitOptions);
    if (r != HIPRTC_SUCCESS) {
        size_t ls = 0;
        hiprtcGetProgramLogSize(prog, &ls);
        std::string log(ls, '\0');
        if (ls) hiprtcGetProgramLog(prog, &log[0]);
        hiprtcDestroyProgram(&prog);
        return fail(PSK_E_JIT, "hipRTC failed for " + name + ": " + log.substr(0, 4000));
    }
    size_t cs = 0;
    hiprtcGetCodeSize(prog, &cs);
    code.resize(cs);
    hiprtcGetCode(prog, code.data());
    hiprtcDestroyProgram(&prog);
    count_jit(false);
    if (!cpath.empty()) {
        std::string tmp = cpath + ".tmp" + std::to_string((long long)std::rand());
        if (FILE* f = std::fopen(tmp.c_str(), "wb")) {
            bool ok = std::fwrite(code.data(), 1, code.size(), f) == code.size();
            std::fclose(f);
            if (ok) std::rename(tmp.c_str(), cpath.c_str());
            else std::remove(tmp.c_str());
        }
    }
    return PSK_OK;
}

}  // namespace psk
