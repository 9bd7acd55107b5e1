// sha256.h -- SHA-256 (FIPS 180-4) of a byte string; host only.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace iso {

void sha256(const uint8_t *msg, size_t len, uint8_t out[32]);

// Incremental form: reset, update any number of times, finish once.
struct Sha256 {
    uint32_t h[8];
    uint64_t nbytes;
    uint8_t buf[64];
    uint32_t nbuf;
    void reset();
    void update(const uint8_t *msg, size_t len);
    void finish(uint8_t out[32]);
};

}  // namespace iso
