// What the launcher stand-ins saw last (sanitizer build of the C-ABI layer).
#pragma once

constexpr int kFailN = 777777;      // a stub reports a launch error for this N

struct StubRecord {
    const char *route = "";
    int fmt = -1, M = 0, N = 0, K = 0;
    long calls = 0;
};

extern StubRecord g_stub;
