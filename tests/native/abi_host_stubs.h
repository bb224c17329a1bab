// Shared between the launcher stand-ins and the host-ABI sanitizer driver.
#pragma once
#include <stdint.h>

enum StubCall { kReplay, kVerify, kFold, kFused, kRewrite, kConv, kSnap, kCommit, kFork, kNumCalls };

struct StubWorld {
    uintptr_t mem = 0;     // fake device address of the registered state memory
    uint64_t total = 0;    // its size in bytes
    uint64_t slots = 0, P = 0, N = 0, esz = 0;
    int batch = 0, rc = 0;
    long calls[kNumCalls] = {};
};
extern StubWorld g_world;
