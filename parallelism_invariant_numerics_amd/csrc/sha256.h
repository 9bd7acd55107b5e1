// sha256.h -- SHA-256 (FIPS 180-4) of a byte string; host only.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace iso {

void sha256(const uint8_t *msg, size_t len, uint8_t out[32]);

}  // namespace iso
