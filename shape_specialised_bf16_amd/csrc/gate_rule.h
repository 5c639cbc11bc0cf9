// gate_rule.h -- the load-time gate's decision on one probe run of a candidate
// (host side).  The statistics come from the check and hash kernels of
// gate.hip; the rule and its log line follow "#004 the same compiler on
// Apple's chips", section "The night the engine chose wrong": a candidate that
// departs from the trusted kernel on a probe is rejected with a log line and
// never timed or picked.  Plain C++ with no HIP call, so that the decision can
// be exercised on the CPU with planted outputs.
#pragma once

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

namespace proj {

// What the check kernels (proj_check_f32 / proj_check_bf16) and the hash
// kernel (proj_hash_out) write for one probe run; the same layout as the
// device's CheckStats in gate.hip.
struct CheckStats {
    uint32_t bad;        // listed-row elements outside the tolerance (not bit-equal on the integer probe)
    uint32_t unwritten;  // elements of rows < M still holding the sentinel
    uint32_t guard;      // elements of the guard rows >= M no longer holding the sentinel
    uint32_t max_err;    // f32 bits of max |y - ref| over the listed rows
    uint32_t max_ref;    // f32 bits of max |ref| over the listed rows
    uint32_t pad;
    uint64_t hash;       // order-independent hash of every element of rows < M (integer probe)
};

inline float gate_bits_f(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

// "" if the run passes the gate; otherwise the line that rejects the
// candidate.  A run fails if any listed-row element is wrong, any row < M was
// left unwritten, any guard row was written, or -- on the integer probe, where
// every summation order gives the same bits, and once the plain kernel's
// whole-output hash `base_hash` is known (have_base) -- the candidate's hash
// of all rows < M differs from it.
inline std::string gate_reject_line(const CheckStats& cs, bool integer, bool have_base, uint64_t base_hash,
                                    int64_t N, int64_t K, int64_t bucket_hi, const std::string& cand, int64_t M)
{
    const bool differs = integer && have_base && cs.hash != base_hash;
    if (!(cs.bad || cs.unwritten || cs.guard || differs)) return "";
    char line[1024];
    snprintf(line, sizeof line,
             "[autotune] proj %lldx%lld %lld rows at %lld: wrong against ref, never picked: %s "
             "(%lld rows%s: max err %.3e of %.3e; %u outside tolerance, %u unwritten, %u written past M%s)",
             (long long)N, (long long)K, (long long)bucket_hi, (long long)bucket_hi, cand.c_str(), (long long)M,
             integer ? ", integer probe" : "", gate_bits_f(cs.max_err), gate_bits_f(cs.max_ref), cs.bad,
             cs.unwritten, cs.guard, differs ? "; whole output differs from the plain kernel's" : "");
    return line;
}

}  // namespace proj
