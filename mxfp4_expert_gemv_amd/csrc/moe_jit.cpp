// moe_jit.cpp -- run-time compilation of the MoE decode kernels for one layer shape (MOE_F_JIT).
//
// The pages' third optimisation compiles its MoE kernels at run time for the actual matrix shapes,
// data types and GPU, in seconds per kernel instead of a long ahead-of-time build of every variant
// (tanhow.com, "NVIDIA 在单台 DGX Spark 上叠加三项优化...", section "三项优化是什么", item 1), and keeps
// the compiled kernels in an on-disk cache (aivibenews.ru, "Три приёма ускорить MoE-инференс на DGX
// Spark без потери GSM8K", section "Три шага по очереди").  Here hipRTC compiles the kernels' device
// code (moe_kernels.h, embedded in the library as text) with the handle's hidden size, expert count,
// top-k, shared-expert count, expert width and input normalisation as compile-time constants, for the
// architecture of the current device.  The code object is cached on disk under a name that carries
// the shape, the architecture and a digest of the source, the options and the kernel list; a later
// create with the same key loads it without compiling.  A failed compile is an error: nothing falls
// back to the ahead-of-time kernels.
#include <hip/hip_runtime.h>
#include <errno.h>
#include <hip/hiprtc.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <chrono>
#include <fstream>
#include <sstream>
#include <string>
#include <vector>

#include "moe_jit.h"
#include "moe_jit_sources.h"

namespace moe {

static uint64_t fnv1a(uint64_t h, const std::string& s) {
    for (unsigned char c : s) {
        h ^= c;
        h *= 0x100000001b3ull;
    }
    return h;
}

static bool make_dirs(const std::string& path) {
    std::string cur;
    for (size_t i = 0; i <= path.size(); ++i) {
        if (i == path.size() || path[i] == '/') {
            if (!cur.empty() && mkdir(cur.c_str(), 0755) != 0 && errno != EEXIST) return false;
        }
        if (i < path.size()) cur += path[i];
    }
    return true;
}

std::string jit_cache_dir() {
    if (const char* d = getenv("MOE_JIT_CACHE_DIR")) return d;
    if (const char* x = getenv("XDG_CACHE_HOME")) return std::string(x) + "/mxfp4_expert_gemv_amd";
    if (const char* h = getenv("HOME")) return std::string(h) + "/.cache/mxfp4_expert_gemv_amd";
    return "/tmp/mxfp4_expert_gemv_amd_cache";
}

static bool read_file(const std::string& path, std::string* out) {
    std::ifstream f(path, std::ios::binary);
    if (!f) return false;
    std::stringstream ss;
    ss << f.rdbuf();
    *out = ss.str();
    return true;
}

// Writes through a temporary name and a rename, so that a reader never sees a partial file.
static bool write_file(const std::string& path, const std::string& data) {
    const std::string tmp = path + ".tmp" + std::to_string(getpid());
    {
        std::ofstream f(tmp, std::ios::binary);
        if (!f) return false;
        f.write(data.data(), (std::streamsize)data.size());
        if (!f) return false;
    }
    return rename(tmp.c_str(), path.c_str()) == 0;
}

moe_status jit_build(const Shape& sh, int max_tokens, bool normalize, bool mfma, JitResult* out) {
    *out = JitResult{};
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return moe_fail(MOE_ERR_HIP, "device query for run-time compilation failed");
    const std::string arch = prop.gcnArchName;
    // the kernel instances of every token count the handle runs
    std::vector<std::string> exprs;
    std::string names[kMaxTokens][kLayerKernels];
    for (int T = 1; T <= max_tokens; ++T) {
        if (!jit_kernel_names(sh, T, mfma, names[T - 1])) return moe_fail(MOE_ERR_UNSUPPORTED, "no kernels for this shape");
        for (const std::string& n : names[T - 1])
            if (!n.empty() && std::find(exprs.begin(), exprs.end(), n) == exprs.end()) exprs.push_back(n);
    }
    std::vector<std::string> opts = {"--offload-arch=" + arch, "-O3", "-std=c++17",
                                     // packed fp32 VALU forms stay disabled, as in the ahead-of-time build
                                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                                     "-DMOE_SHAPE_H=" + std::to_string(sh.H), "-DMOE_SHAPE_E=" + std::to_string(sh.E),
                                     "-DMOE_SHAPE_K=" + std::to_string(sh.k), "-DMOE_SHAPE_S=" + std::to_string(sh.S),
                                     "-DMOE_SHAPE_I=" + std::to_string(sh.I),
                                     std::string("-DMOE_SHAPE_NORM=") + (normalize ? "1" : "0")};
    uint64_t key = fnv1a(0xcbf29ce484222325ull, kJitSourceDigest);
    for (const std::string& o : opts) key = fnv1a(key, o + "\n");
    for (const std::string& e : exprs) key = fnv1a(key, e + "\n");
    std::string arch_tag = arch;
    for (char& c : arch_tag)
        if (c == ':' || c == '+' || c == '/') c = c == '+' ? 'p' : '_';
    char base[256];
    snprintf(base, sizeof base, "moe_h%d_e%d_k%d_s%d_i%d_n%d_t%d%s_%s_%016llx", sh.H, sh.E, sh.k, sh.S, sh.I,
             normalize ? 1 : 0, max_tokens, mfma ? "_mf" : "", arch_tag.c_str(), (unsigned long long)key);
    const std::string dir = jit_cache_dir();
    const std::string co_path = dir + "/" + base + ".co", names_path = dir + "/" + base + ".names";
    snprintf(out->path, sizeof out->path, "%s", co_path.c_str());

    std::string code, lowered_text;
    std::vector<std::string> lowered(exprs.size());
    if (read_file(co_path, &code) && read_file(names_path, &lowered_text)) {
        std::istringstream ls(lowered_text);
        std::string line;
        size_t i = 0;
        while (std::getline(ls, line) && i < exprs.size()) {
            const size_t tab = line.find('\t');
            if (tab == std::string::npos || line.substr(0, tab) != exprs[i]) break;
            lowered[i++] = line.substr(tab + 1);
        }
        out->from_cache = i == exprs.size() && !code.empty();
    }
    if (!out->from_cache) {
        std::vector<const char*> hdr_texts(kJitHeaderTexts, kJitHeaderTexts + kJitHeaderCount);
        std::vector<const char*> hdr_names(kJitHeaderNames, kJitHeaderNames + kJitHeaderCount);
        hiprtcProgram prog;
        if (hiprtcCreateProgram(&prog, "#include \"moe_kernels.h\"\n", "moe_jit.hip", kJitHeaderCount,
                                hdr_texts.data(), hdr_names.data()) != HIPRTC_SUCCESS)
            return moe_fail(MOE_ERR_HIP, "hiprtcCreateProgram failed");
        for (const std::string& e : exprs) hiprtcAddNameExpression(prog, e.c_str());
        std::vector<const char*> copts;
        for (const std::string& o : opts) copts.push_back(o.c_str());
        const auto t0 = std::chrono::steady_clock::now();
        const hiprtcResult r = hiprtcCompileProgram(prog, (int)copts.size(), copts.data());
        out->compile_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
        if (r != HIPRTC_SUCCESS) {
            size_t n = 0;
            hiprtcGetProgramLogSize(prog, &n);
            std::string log(n, '\0');
            if (n) hiprtcGetProgramLog(prog, &log[0]);
            hiprtcDestroyProgram(&prog);
            return moe_fail(MOE_ERR_HIP, "run-time compilation failed (%s): %.300s", hiprtcGetErrorString(r),
                            log.c_str());
        }
        size_t n = 0;
        hiprtcGetCodeSize(prog, &n);
        code.assign(n, '\0');
        hiprtcGetCode(prog, &code[0]);
        lowered_text.clear();
        for (size_t i = 0; i < exprs.size(); ++i) {
            const char* lo = nullptr;
            if (hiprtcGetLoweredName(prog, exprs[i].c_str(), &lo) != HIPRTC_SUCCESS || !lo) {
                hiprtcDestroyProgram(&prog);
                return moe_fail(MOE_ERR_HIP, "no lowered name for %s", exprs[i].c_str());
            }
            lowered[i] = lo;
            lowered_text += exprs[i] + "\t" + lo + "\n";
        }
        hiprtcDestroyProgram(&prog);
        // a cache that cannot be written only costs the next create a compile
        if (make_dirs(dir)) {
            if (write_file(co_path, code)) (void)write_file(names_path, lowered_text);
        }
    }
    if (hipModuleLoadData(&out->module, code.data()) != hipSuccess) {
        (void)hipGetLastError();
        out->module = nullptr;
        return moe_fail(MOE_ERR_HIP, "hipModuleLoadData of the run-time compiled kernels failed");
    }
    for (int T = 1; T <= max_tokens; ++T)
        for (int k = 0; k < kLayerKernels; ++k) {
            const std::string& n = names[T - 1][k];
            if (n.empty()) continue;
            const size_t i = (size_t)(std::find(exprs.begin(), exprs.end(), n) - exprs.begin());
            if (hipModuleGetFunction(&out->kernels.fn[T - 1][k], out->module, lowered[i].c_str()) != hipSuccess) {
                (void)hipGetLastError();
                jit_release(out);
                return moe_fail(MOE_ERR_HIP, "kernel %s missing from the run-time compiled module", n.c_str());
            }
        }
    return MOE_OK;
}

void jit_release(JitResult* r) {
    if (r->module) (void)hipModuleUnload(r->module);
    r->module = nullptr;
}

}  // namespace moe
