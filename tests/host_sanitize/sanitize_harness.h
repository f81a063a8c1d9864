// Shared between the launcher stand-ins and the boundary driver of the host
// sanitizer build: the buffers a call hands the library (so the stand-ins can
// check every extent a kernel would touch), and the launch and failure counts.
#pragma once

#include <stddef.h>

void harness_register(const char* name, const void* p, size_t bytes);
void harness_clear();
int harness_launches();
int harness_failures();
