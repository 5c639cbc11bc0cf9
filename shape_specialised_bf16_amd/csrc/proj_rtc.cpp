// proj_rtc.cpp -- compile helper of libproj: one HIP source file to one code
// object with hipRTC.  libproj starts several of these as child processes to
// compile the modules of a plan at the same time (hipRTC compiles one program
// at a time per process).  Touches no GPU.
//
//     proj_rtc <arch> <source.hip> <out.co>
//
// Exit status 0 on success (out.co written whole, through a temporary file
// renamed into place); 1 if the compilation failed (hipRTC's log on stderr);
// 2 on a usage or file error.
#include <cstdio>
#include <fstream>
#include <iterator>
#include <string>
#include <vector>

#include "rtc.h"

int main(int argc, char** argv)
{
    if (argc != 4) {
        fprintf(stderr, "usage: %s <arch> <source.hip> <out.co>\n", argv[0]);
        return 2;
    }
    std::ifstream in(argv[2], std::ios::binary);
    if (!in) {
        fprintf(stderr, "proj_rtc: cannot read %s\n", argv[2]);
        return 2;
    }
    const std::string src((std::istreambuf_iterator<char>(in)), std::istreambuf_iterator<char>());
    std::string name = argv[2];
    const size_t slash = name.rfind('/');
    if (slash != std::string::npos) name = name.substr(slash + 1);
    std::vector<char> code;
    std::string log;
    if (proj::rtc_compile(src, argv[1], name, &code, &log) != 0) {
        fprintf(stderr, "%s\n", log.c_str());
        return 1;
    }
    const std::string tmp = std::string(argv[3]) + ".tmp";
    {
        std::ofstream out(tmp, std::ios::binary);
        if (!out || !out.write(code.data(), (std::streamsize)code.size())) {
            fprintf(stderr, "proj_rtc: cannot write %s\n", tmp.c_str());
            std::remove(tmp.c_str());
            return 2;
        }
    }
    if (std::rename(tmp.c_str(), argv[3]) != 0) {
        fprintf(stderr, "proj_rtc: cannot rename %s\n", tmp.c_str());
        std::remove(tmp.c_str());
        return 2;
    }
    return 0;
}
