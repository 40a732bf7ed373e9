// Internal: the static device scratch behind jpa_forward_scratch
// (jpa_scratch.hip).  Not part of the public ABI.
#ifndef JPA_SCRATCH_H
#define JPA_SCRATCH_H

#include <stddef.h>

// Bytes of the per-device scratch array.
size_t jpa_scratch_bytes();
// Device address of the current device's scratch array (looked up once per
// device); returns the hipError_t of the lookup as an int.
int jpa_scratch_address(void** ptr);

#endif
