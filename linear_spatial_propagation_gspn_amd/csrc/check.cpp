// check.cpp -- the registry of the host-side launch checker (check.hpp);
// compiled only into libgspn_check.so, with its C entry points below.
#include "check.hpp"

#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <deque>
#include <mutex>
#include <string>
#include <vector>

#ifndef GSPN_CHECK_LAUNCHES
#error "check.cpp belongs to the host-only checking build"
#endif

namespace gspn {
namespace check {
namespace {

constexpr int kMaxReported = 32;
constexpr int64_t kLdsBytes = 160 * 1024;  // LDS one workgroup may hold on gfx950

struct State {
    std::mutex mu;
    std::vector<Region> regions;  // sorted by lo, disjoint
    std::deque<std::string> names;  // stable addresses: the regions point into them
    std::vector<std::string> log;
    std::vector<std::string> reported;
    int64_t violations = 0;
    int64_t accesses = 0;
    int64_t launches = 0;
    std::string pending;  // kernel replayed and not yet launched
    int pending_threads = 0;
    int64_t pending_lds = 0;
};

State& state() {
    static State s;
    return s;
}

// A kernel expression as the launch macro spells it, "(name<args>)", down to its name.
std::string base_name(const char* k) {
    std::string s(k);
    while (!s.empty() && (s.front() == '(' || s.front() == ' ')) s.erase(s.begin());
    const size_t lt = s.find('<');
    if (lt != std::string::npos) s.erase(lt);
    while (!s.empty() && (s.back() == ')' || s.back() == ' ')) s.pop_back();
    return s;
}

void report_locked(State& s, const std::string& msg) {
    ++s.violations;
    if (static_cast<int>(s.reported.size()) < kMaxReported) s.reported.push_back(msg);
}

}  // namespace

Region region_of(const void* p, const char* kernel, const char* what) {
    State& s = state();
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    {
        std::lock_guard<std::mutex> lock(s.mu);
        auto it = std::upper_bound(s.regions.begin(), s.regions.end(), a,
                                   [](uint64_t v, const Region& r) { return v < r.lo; });
        if (it != s.regions.begin()) {
            --it;
            if (a >= it->lo && a < it->hi) return *it;
        }
    }
    violation(kernel, what, "pointer %p lies in no registered buffer", p);
    return Region{};
}

void violation(const char* kernel, const char* what, const char* fmt, ...) {
    char buf[512];
    int n = snprintf(buf, sizeof buf, "%s: %s: ", kernel, what);
    va_list ap;
    va_start(ap, fmt);
    if (n > 0 && n < static_cast<int>(sizeof buf)) vsnprintf(buf + n, sizeof buf - n, fmt, ap);
    va_end(ap);
    State& s = state();
    std::lock_guard<std::mutex> lock(s.mu);
    report_locked(s, buf);
}

void count_accesses(int64_t n) {
    State& s = state();
    std::lock_guard<std::mutex> lock(s.mu);
    s.accesses += n;
}

void replayed(const char* kernel, int max_threads, int64_t static_lds) {
    State& s = state();
    std::lock_guard<std::mutex> lock(s.mu);
    s.pending = base_name(kernel);
    s.pending_threads = max_threads;
    s.pending_lds = static_lds;
}

void launched(const char* kernel, dim3 grid, dim3 block, size_t dyn_lds) {
    State& s = state();
    std::lock_guard<std::mutex> lock(s.mu);
    ++s.launches;
    char line[512];
    snprintf(line, sizeof line, "%s grid=%u block=%u lds=%zu+%lld", kernel, grid.x, block.x, dyn_lds,
             static_cast<long long>(s.pending_lds));
    s.log.push_back(line);
    if (s.pending != base_name(kernel)) {
        report_locked(s, std::string(kernel) + ": launched without a host replay of its accesses");
    } else {
        const uint64_t threads = static_cast<uint64_t>(block.x) * block.y * block.z;
        if (grid.x < 1 || grid.y < 1 || grid.z < 1 || grid.y > 65535 || grid.z > 65535)
            report_locked(s, std::string(line) + ": grid out of range");
        if (threads < 1 || threads > static_cast<uint64_t>(s.pending_threads))
            report_locked(s, std::string(line) + ": block exceeds the kernel's launch bound");
        if (static_cast<int64_t>(dyn_lds) + s.pending_lds > kLdsBytes)
            report_locked(s, std::string(line) + ": LDS beyond 160 KiB");
    }
    s.pending.clear();
}

}  // namespace check
}  // namespace gspn

using gspn::check::State;

extern "C" {

// Forgets every buffer, launch and violation.
void gspn_check_reset(void) {
    State& s = gspn::check::state();
    std::lock_guard<std::mutex> lock(s.mu);
    s.regions.clear();
    s.names.clear();
    s.log.clear();
    s.reported.clear();
    s.violations = s.accesses = s.launches = 0;
    s.pending.clear();
}

// Registers buffer [base, base + bytes) under name; 0, or -1 if it overlaps
// one already registered or is empty.
int gspn_check_add_buffer(const char* name, uint64_t base, uint64_t bytes) {
    State& s = gspn::check::state();
    std::lock_guard<std::mutex> lock(s.mu);
    if (bytes == 0) return -1;
    for (const auto& r : s.regions)
        if (base < r.hi && r.lo < base + bytes) return -1;
    s.names.emplace_back(name);
    gspn::check::Region r{base, base + bytes, s.names.back().c_str()};
    s.regions.insert(std::upper_bound(s.regions.begin(), s.regions.end(), r,
                                      [](const gspn::check::Region& a, const gspn::check::Region& b) {
                                          return a.lo < b.lo;
                                      }),
                     r);
    return 0;
}

int64_t gspn_check_violations(void) { return gspn::check::state().violations; }
int64_t gspn_check_accesses(void) { return gspn::check::state().accesses; }
int64_t gspn_check_launches(void) { return gspn::check::state().launches; }

// Writes the launch log and the first violations, one per line, into buf
// (NUL-terminated, truncated to cap bytes); returns the full length.
int64_t gspn_check_report(char* buf, int64_t cap) {
    State& s = gspn::check::state();
    std::lock_guard<std::mutex> lock(s.mu);
    std::string out;
    for (const auto& l : s.log) out += "launch " + l + "\n";
    for (const auto& v : s.reported) out += "violation " + v + "\n";
    if (buf && cap > 0) {
        const size_t n = std::min(out.size(), static_cast<size_t>(cap - 1));
        std::copy(out.begin(), out.begin() + n, buf);
        buf[n] = '\0';
    }
    return static_cast<int64_t>(out.size());
}

}  // extern "C"
