// rtc.h -- one hipRTC compilation (HIP source text -> code object), shared by
// libproj and its compile helper executable proj_rtc.
#pragma once

#include <string>
#include <vector>

namespace proj {

// The hipRTC options besides --offload-arch, and the same as one line of text
// (part of the compiled-module cache key).  -packed-fp32-ops is switched off:
// no packed f32 ALU instructions in any kernel.
extern const char* const kRtcOptions[];
extern const int kRtcNumOptions;
extern const char* const kRtcOptionText;

// Compile `src` for `arch` (e.g. "gfx950").  Returns 0 and fills `code`, or -1
// with hipRTC's log (or the failing call) in `log`.  Needs no GPU.
int rtc_compile(const std::string& src, const std::string& arch, const std::string& name, std::vector<char>* code,
                std::string* log);

}  // namespace proj
