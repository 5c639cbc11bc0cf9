// rtc.cpp -- one hipRTC compilation, for libproj and for proj_rtc.
#include "rtc.h"

#include <hip/hiprtc.h>

namespace proj {

const char* const kRtcOptions[] = {"-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"};
const int kRtcNumOptions = (int)(sizeof kRtcOptions / sizeof kRtcOptions[0]);
const char* const kRtcOptionText = "-O3 -std=c++17 -Xclang -target-feature -Xclang -packed-fp32-ops";

int rtc_compile(const std::string& src, const std::string& arch, const std::string& name, std::vector<char>* code,
                std::string* log)
{
    hiprtcProgram prog;
    hiprtcResult r = hiprtcCreateProgram(&prog, src.c_str(), name.c_str(), 0, nullptr, nullptr);
    if (r != HIPRTC_SUCCESS) {
        *log = std::string("hiprtcCreateProgram: ") + hiprtcGetErrorString(r);
        return -1;
    }
    const std::string arch_opt = "--offload-arch=" + arch;
    std::vector<const char*> opts = {arch_opt.c_str()};
    for (int i = 0; i < kRtcNumOptions; ++i) opts.push_back(kRtcOptions[i]);
    r = hiprtcCompileProgram(prog, (int)opts.size(), opts.data());
    if (r != HIPRTC_SUCCESS) {
        size_t ls = 0;
        hiprtcGetProgramLogSize(prog, &ls);
        std::string l(ls, '\0');
        if (ls) hiprtcGetProgramLog(prog, &l[0]);
        while (!l.empty() && l.back() == '\0') l.pop_back();
        *log = std::string(hiprtcGetErrorString(r)) + (l.empty() ? "" : ": " + l);
        hiprtcDestroyProgram(&prog);
        return -1;
    }
    size_t cs = 0;
    hiprtcGetCodeSize(prog, &cs);
    code->assign(cs, 0);
    r = hiprtcGetCode(prog, code->data());
    hiprtcDestroyProgram(&prog);
    if (r != HIPRTC_SUCCESS || cs == 0) {
        *log = "hiprtcGetCode returned no code object";
        return -1;
    }
    return 0;
}

}  // namespace proj
